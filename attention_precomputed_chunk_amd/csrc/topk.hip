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
// T the lowest indices are taken. The k winners are written in index order
// and sorted by key, descending, with a stable LSD radix sort over the bits
// where they differ, which leaves equal keys in index order: the output is
// ordered by (value descending, index ascending).
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
    // lane w < 16 holds wave w's total; an exclusive scan of those over the
    // lanes, read at lane `wave`, is the sum of the waves before this one
    int t = lane < kTopkWaves ? wave_tot[lane] : 0;
#pragma unroll
    for (int off = 1; off < kTopkWaves; off <<= 1) {
        const int y = __shfl_up(t, off);
        if (lane >= off)
            t += y;
    }
    const int before = __shfl(t, wave) - wave_tot[wave];
    __syncthreads();
    return x + before;
}

__device__ __forceinline__ void topk_body(const TopkDesc td)
{
    __shared__ __attribute__((aligned(16))) uint32_t keys[kTopkLdsKeys];   // then the sort's second buffer
    __shared__ __attribute__((aligned(16))) uint32_t whist[kTopkWaves][256];
    __shared__ __attribute__((aligned(16))) unsigned long long sel[kTopkMaxK];
    __shared__ int wave_tot[kTopkWaves];
    __shared__ uint32_t red_min[kTopkWaves], red_max[kTopkWaves];
    __shared__ uint32_t s_digit;
    __shared__ int s_above;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = td.n, k = td.k;
    const bool in_lds = n <= kTopkLdsKeys;
    auto key_at = [&](int i) -> uint32_t { return in_lds ? keys[i] : order_key(td.value[i]); };

    // keys, and the common prefix of all of them (eight loads in flight per
    // thread)
    uint32_t mn = 0xFFFFFFFFu, mx = 0u;
    constexpr int kLoadBatch = 8;
    for (int i0 = tid; i0 < n; i0 += kLoadBatch * kTopkThreads) {
        float v[kLoadBatch];
#pragma unroll
        for (int j = 0; j < kLoadBatch; ++j) {
            const int i = i0 + j * kTopkThreads;
            v[j] = i < n ? td.value[i] : 0.f;
        }
#pragma unroll
        for (int j = 0; j < kLoadBatch; ++j) {
            const int i = i0 + j * kTopkThreads;
            if (i < n) {
                const uint32_t kk = order_key(v[j]);
                if (in_lds)
                    keys[i] = kk;
                mn = min(mn, kk);
                mx = max(mx, kk);
            }
        }
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
            // lane l owns digits 255-4l .. 252-4l (scanning from the top),
            // four adjacent bins read as one 16-byte word per wave
            int c[4] = {0, 0, 0, 0}, tot = 0;
#pragma unroll
            for (int w = 0; w < kTopkWaves; ++w) {
                const uint4 h4 = *reinterpret_cast<const uint4 *>(&whist[w][252 - 4 * lane]);
                c[0] += (int)h4.w;   // digit 255 - 4 lane
                c[1] += (int)h4.z;
                c[2] += (int)h4.y;
                c[3] += (int)h4.x;   // digit 252 - 4 lane
            }
#pragma unroll
            for (int q = 0; q < 4; ++q)
                tot += c[q];
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

    // The k winners in index order: thread t scans indices [t*chunk, ...),
    // counting keys above T and keys equal to T; scans of both counts place
    // every winner and decide which ties are taken (the first `remaining` in
    // index order).
    // (Keys in LDS: chunks of a multiple of 4 keys, read 16 bytes at a time.)
    const int chunk0 = (n + kTopkThreads - 1) / kTopkThreads;
    const int chunk = in_lds ? (chunk0 + 3) & ~3 : chunk0;
    const int b = min(n, tid * chunk), e = min(n, b + chunk);
    int gt = 0, eq = 0;
    auto count = [&](uint32_t kk) {
        gt += kk > T ? 1 : 0;
        eq += kk == T ? 1 : 0;
    };
    if (in_lds) {
        for (int i = b; i < e; i += 4) {
            const uint4 q = *reinterpret_cast<const uint4 *>(&keys[i]);
            count(q.x);
            if (i + 1 < e)
                count(q.y);
            if (i + 2 < e)
                count(q.z);
            if (i + 3 < e)
                count(q.w);
        }
    } else {
        for (int i = b; i < e; ++i)
            count(key_at(i));
    }
    const int gt_before = block_inclusive_scan(gt, wave_tot) - gt;
    const int eq_before = block_inclusive_scan(eq, wave_tot) - eq;
    int taken = min(eq_before, remaining);   // ties taken before this thread's chunk
    int pos = gt_before + taken;
    auto place = [&](uint32_t kk, int i) {
        if (kk > T || (kk == T && taken < remaining)) {
            sel[pos++] = ((unsigned long long)kk << 32) | (unsigned int)i;
            taken += kk == T ? 1 : 0;
        }
    };
    if (in_lds) {
        for (int i = b; i < e; i += 4) {
            const uint4 q = *reinterpret_cast<const uint4 *>(&keys[i]);
            place(q.x, i);
            if (i + 1 < e)
                place(q.y, i + 1);
            if (i + 2 < e)
                place(q.z, i + 2);
            if (i + 3 < e)
                place(q.w, i + 3);
        }
    } else {
        for (int i = b; i < e; ++i)
            place(key_at(i), i);
    }
    __syncthreads();

    // Stable LSD radix sort of the k winners by key, descending (bin = 255 -
    // digit), over the 8-bit digits below the common prefix of the largest
    // key and T; equal keys keep index order. Wave w ranks the entries
    // [w*S, (w+1)*S) in rounds of 64: within a round the lanes holding the
    // same digit find each other with 8 ballots, and a wave-private count per
    // bin carries the rank across rounds. The counts then become each
    // (bin, wave)'s first slot, in bin order then wave order, and every entry
    // moves there. The sort ping-pongs between sel and `keys`, free once the
    // winners are picked (8192 64-bit entries either way).
    unsigned long long *src = sel;
    unsigned long long *dst = reinterpret_cast<unsigned long long *>(keys);
    const int sig = (T == mx) ? 0 : 32 - __clz((int)(T ^ mx));   // bits that differ among the winners
    const int S = ((k + kTopkWaves - 1) / kTopkWaves + 63) / 64 * 64;   // entries per wave
    const int rounds = S / 64;   // <= kTopkMaxK / kTopkWaves / 64 = 8
    const unsigned long long below = (1ull << lane) - 1ull;
    for (int shift = 0; shift < sig; shift += 8) {
        for (int q = lane; q < 256; q += 64)
            whist[wave][q] = 0;
        unsigned long long ent[kTopkMaxK / kTopkWaves / 64];
        int bin[kTopkMaxK / kTopkWaves / 64], rank[kTopkMaxK / kTopkWaves / 64];
#pragma unroll
        for (int r = 0; r < kTopkMaxK / kTopkWaves / 64; ++r) {
            if (r < rounds) {   // wave-uniform
                const int i = wave * S + r * 64 + lane;
                const bool valid = i < k;
                ent[r] = valid ? src[i] : 0ull;
                bin[r] = 255 - (int)((ent[r] >> (32 + shift)) & 255u);
                unsigned long long peers = __ballot(valid);
#pragma unroll
                for (int bit = 0; bit < 8; ++bit) {
                    const unsigned long long on = __ballot((bin[r] >> bit) & 1);
                    peers &= ((bin[r] >> bit) & 1) ? on : ~on;
                }
                const int before = __popcll(peers & below);
                rank[r] = (int)whist[wave][bin[r]] + before;   // read by every lane before the leader adds
                if (valid && (peers >> lane) == 1ull)      // the highest lane of its digit group
                    whist[wave][bin[r]] += (uint32_t)(before + 1);
            }
        }
        __syncthreads();
        // (bin, wave) -> first slot: bins in order, waves in order within a bin
        int tot = 0;
        uint32_t c[kTopkWaves];
        if (tid < 256) {
#pragma unroll
            for (int w = 0; w < kTopkWaves; ++w)
                c[w] = whist[w][tid];
#pragma unroll
            for (int w = 0; w < kTopkWaves; ++w)
                tot += (int)c[w];
        }
        int base = block_inclusive_scan(tot, wave_tot) - tot;
        if (tid < 256) {
#pragma unroll
            for (int w = 0; w < kTopkWaves; ++w) {
                whist[w][tid] = (uint32_t)base;
                base += (int)c[w];
            }
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < kTopkMaxK / kTopkWaves / 64; ++r)
            if (r < rounds && wave * S + r * 64 + lane < k)
                dst[whist[wave][bin[r]] + rank[r]] = ent[r];
        __syncthreads();
        unsigned long long *t = src;
        src = dst;
        dst = t;
    }
    for (int i = tid; i < k; i += kTopkThreads)
        td.idx[i] = (int32_t)(src[i] & 0xFFFFFFFFull);
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
