// Pass 1 of the attention (the row log-sum-exp) as a kernel of its own, for
// gfx950 (CDNA4), run before pass 2 on the same work items (TurboRAG summary,
// the causal attention equation; CacheBlend summary, the selective-recompute
// listing's softmax over every key):
//   lse_j = log sum_i exp(q_j . k_i / sqrt(d))   over the keys visible to row j
// Each work item covers one range of its row block's key tiles and stores,
// per packed row, the partial state of that range: the largest raw score m
// and l = sum_i exp2((s_ji - m) c) with c = log2(e) / sqrt(d). Pass 2 merges
// the states of its block's ranges in range order, so every range of a block
// uses the same lse, and lse_j / ln 2 = m c + log2 l.
//
// Why a separate kernel: a wave issues its vector and matrix instructions in
// order, and in the one-wave-per-SIMD kernel the two barely overlap; a second
// wave on the SIMD supplies the overlap. Pass 2 needs the output accumulators
// of all its rows and so fills a SIMD's registers with one wave, but pass 1
// needs only Q and two numbers per row: here 8 waves (two per SIMD) share
// each staged K tile, and each wave takes a run of consecutive row tiles of
// the item's block (lse_rows). Each wave runs a body compiled for its own
// number of row tiles (0 .. 4), so no padded tile is computed; every body
// meets the same barriers.
//
// The arithmetic per key tile is the one-wave kernel's pass 1: scores on the
// matrix cores (S^T = K Q^T, layout in attn_bf16_common.h), the running
// maximum and sum of exp2 per row, with unmasked tiles summed against a
// reference maximum and the exact maximum taken again only when a sum leaves
// float32's comfortable range (see kLseRescaleBound).
#include <type_traits>

#include "attn_bf16_common.h"

namespace crkv {

// SPLIT: only the waves with srank >= 0 move key tiles (the others only
// score); otherwise every thread moves its share (srank unused).
// The wave's row tiles are first .. first + R - 1 of the block.
template <int D, int R, bool KV8, bool SPLIT, typename Stg>
__device__ __forceinline__ void lse_body(const AttnArgs &a, const ItemDesc &it, const ProbDesc &pr, const Stg &stg,
                                         unsigned char (*lds_k)[kTileK<D / 8>],
                                         unsigned char (*lds_kl)[KV8 ? kTileK<D / 8> : 16], int first, int lane,
                                         int srank)
{
    constexpr int KS = D / 32;
    constexpr int NCH = D / 8;
    constexpr int RR = R > 0 ? R : 1;
    const int li = lane & 15, lg = lane >> 4;
    const int G = a.G;
    const float c = a.c_log2;
    const int n_kt = it.n_ktiles;
    const int kt0 = it.kt_begin;

    int row_pos[RR];
    bf16x8 qf[RR][KS];
    float row_m[RR], row_l[RR];
#pragma unroll
    for (int i = 0; i < R; ++i) {
        load_q_rows<KS>(pr, it, G, it.tile_begin + first + i, li, lg, qf[i], row_pos[i]);
        row_m[i] = -INFINITY;
        row_l[i] = 0.f;
    }
    const int wave_min_pos = pr.pos0 + ((it.tile_begin + first) * kRowTile) / G;

    auto k_off = [&](int sub, int ks) { return k_frag_off<NCH>(li, lg, sub, ks); };
    auto load_kf = [&](int buf, bf16x8 (&kf)[2][KS], bf16x8 (&kfl)[KV8 ? 2 : 1][KS]) {
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                kf[sub][ks] = *reinterpret_cast<const bf16x8 *>(&lds_k[buf][k_off(sub, ks)]);
                if constexpr (KV8)
                    kfl[sub][ks] = *reinterpret_cast<const bf16x8 *>(&lds_kl[buf][k_off(sub, ks)]);
            }
    };
    auto qk = [&](const bf16x8 (&kf)[2][KS], const bf16x8 (&kfl)[KV8 ? 2 : 1][KS], int i, f32x4 &s0, f32x4 &s1) {
        s0 = f32x4{0.f, 0.f, 0.f, 0.f};
        s1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[0][ks], qf[i][ks], s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[1][ks], qf[i][ks], s1, 0, 0, 0);
            if constexpr (KV8) {
                s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfl[0][ks], qf[i][ks], s0, 0, 0, 0);
                s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfl[1][ks], qf[i][ks], s1, 0, 0, 0);
            }
        }
    };
    // Exact running maximum and rescaled sum (masked tiles, a row's first
    // tile, and the fallback of the reference path).
    auto tile_exact = [&](TileSR kt, int buf, auto mask_tag) {
        constexpr bool MASK = decltype(mask_tag)::value;
        bf16x8 kf[2][KS], kfl[KV8 ? 2 : 1][KS];
        load_kf(buf, kf, kfl);
#pragma unroll
        for (int i = 0; i < R; ++i) {
            f32x4 s0, s1;
            qk(kf, kfl, i, s0, s1);
            if constexpr (MASK) {
                const int lim = min(kt.n_valid - 1, row_pos[i] - kt.key0);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (acc_key(lg, 0, e) > lim)
                        s0[e] = -INFINITY;
                    if (acc_key(lg, 1, e) > lim)
                        s1[e] = -INFINITY;
                }
            }
            const float tmax = fmaxf(fmaxf(fmaxf(row_m[i], s0[0]), fmaxf(s0[1], s0[2])),
                                     fmaxf(fmaxf(s0[3], s1[0]), fmaxf(fmaxf(s1[1], s1[2]), s1[3])));
            const float mc = ((tmax == -INFINITY) ? 0.f : tmax) * c;
            float sum = exp2_hw(__builtin_fmaf(s0[0], c, -mc)) + exp2_hw(__builtin_fmaf(s1[0], c, -mc));
#pragma unroll
            for (int e = 1; e < 4; ++e)
                sum += exp2_hw(__builtin_fmaf(s0[e], c, -mc)) + exp2_hw(__builtin_fmaf(s1[e], c, -mc));
            row_l[i] = __builtin_fmaf(row_l[i], exp2_hw(__builtin_fmaf(row_m[i], c, -mc)), sum);
            row_m[i] = tmax;
        }
    };
    // Unmasked tile against the current maxima; false (nothing changed) when
    // some row needs its maximum taken again.
    auto tile_ref = [&](int buf) -> bool {
        bf16x8 kf[2][KS], kfl[KV8 ? 2 : 1][KS];
        load_kf(buf, kf, kfl);
        float sum[RR];
        bool big = false;
#pragma unroll
        for (int i = 0; i < R; ++i) {
            f32x4 s0, s1;
            qk(kf, kfl, i, s0, s1);
            const float mc = row_m[i] * c;
            float e[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                e[j] = exp2_hw(__builtin_fmaf(s0[j], c, -mc));
                e[4 + j] = exp2_hw(__builtin_fmaf(s1[j], c, -mc));
            }
            sum[i] = ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
            big |= sum[i] > kLseRescaleBound;
        }
        if (__builtin_amdgcn_ballot_w64(big))
            return false;
#pragma unroll
        for (int i = 0; i < R; ++i)
            row_l[i] += sum[i];
        return true;
    };

    auto stage_load = [&](TileSR kt) {
        if constexpr (KV8)
            return stg.load(kt, it.kv_head, a.H_kv);
        else
            return stg.load(kt, it.kv_head);
    };
    auto stage_store = [&](const auto &st, int buf) {
        if constexpr (KV8)
            stg.store(st, lds_k[buf], lds_kl[buf], nullptr);
        else
            stg.store(st, lds_k[buf], nullptr);
    };
    // Two key tiles per barrier: step g scores tiles 2g and 2g + 1 from one
    // pair of LDS buffers while tiles 2g + 2 and 2g + 3 are loaded into
    // registers and then stored into the other pair; descriptors run two
    // tiles further ahead. (One tile per barrier left each step's load
    // latency and barrier exposed; deeper register prefetch and a software-
    // pipelined form that scored the next row tile under this one's
    // exponentials measured slower.)
    auto desc = [&](int tt) { return load_tile(pr.tiles, kt0 + min(tt, n_kt - 1), lane); };
    auto run = [&](TileSR kt, int buf) {
        if constexpr (R > 0) {
            const bool need_mask = (kt.n_valid < kKeyTile) || (kt.key0 + kt.n_valid - 1 > wave_min_pos);
            if (need_mask)
                tile_exact(kt, buf, std::true_type{});
            else if (!tile_ref(buf))
                tile_exact(kt, buf, std::false_type{});
        }
    };
    const bool stages = !SPLIT || srank >= 0;   // wave-uniform
    TileSR c0 = to_sr(desc(0)), c1 = to_sr(desc(1));
    if (stages) {
        stage_store(stage_load(c0), 0);
        if (n_kt > 1)
            stage_store(stage_load(c1), 1);
    }
    uint32_t raw0 = desc(2), raw1 = desc(3);
    __syncthreads();
    const int n_steps = (n_kt + 1) / 2;
    for (int g = 0; g < n_steps; ++g) {
        const int base = (g & 1) * 2;
        const int ta = 2 * g + 2, tb = 2 * g + 3;   // tiles loaded during this step
        const TileSR s0 = to_sr(raw0), s1 = to_sr(raw1);
        raw0 = desc(ta + 2);
        raw1 = desc(tb + 2);
        decltype(stage_load(s0)) sa, sb;
        if (stages && ta < n_kt)
            sa = stage_load(s0);
        if (stages && tb < n_kt)
            sb = stage_load(s1);
        run(c0, base);
        if (2 * g + 1 < n_kt)
            run(c1, base + 1);
        if (stages && ta < n_kt)
            stage_store(sa, base ^ 2);
        if (stages && tb < n_kt)
            stage_store(sb, (base ^ 2) + 1);
        __syncthreads();
        c0 = s0;
        c1 = s1;
    }

    // The four lane groups of a row hold partial (max, sum) states: combine
    // them into the range's state (rows that see no key of the range keep
    // (-inf, 0); padded rows are never read).
    const gptr<f32x2> state = as_global(reinterpret_cast<f32x2 *>(a.state)) + (size_t)it.state + (size_t)it.range * a.cap_rows;
#pragma unroll
    for (int i = 0; i < R; ++i) {
        float m = row_m[i], l = row_l[i];
        merge_state(m, l, __shfl_xor(m, 16), __shfl_xor(l, 16), c);
        merge_state(m, l, __shfl_xor(m, 32), __shfl_xor(l, 32), c);
        const int local = (first + i) * kRowTile + li;   // packed row inside the item's block
        if (lg == 0)
            state[local] = f32x2{m, l};
    }
}

// Row tiles per wave. SIMD s (waves s and s + 4) takes n / 4 row tiles of
// the block's n, one more for s < n % 4. Of a SIMD's two waves the first
// keeps issue priority and, with equal shares, finishes its step while the
// second has done about half of its own and then runs alone at a lone
// wave's rate; the first wave therefore takes about two thirds of the
// SIMD's row tiles (at most 4), so that both run until the barrier. Waves
// hold consecutive row tiles, in wave order.
__device__ __forceinline__ int lse_rows(int n, int wave)
{
    const int s = wave & 3;
    const int sc = n / 4 + (s < n % 4 ? 1 : 0);
    const int first = min(kLseMaxRowTilesPerWave, (2 * sc + 1) / 3);
    return wave < 4 ? first : sc - first;
}

// With n % 4 in 1 .. 3, SIMDs 0 .. n % 4 - 1 hold one row tile more than the
// others; then (bf16) two waves of the lighter SIMDs move every key tile and
// the busier SIMDs only score.
template <int D, bool KV8, bool SPLIT>
__device__ __forceinline__ void lse_dispatch(const AttnArgs &a, const ItemDesc &it, const ProbDesc &pr,
                                             unsigned char (*lds_k)[kTileK<D / 8>],
                                             unsigned char (*lds_kl)[KV8 ? kTileK<D / 8> : 16], int wave,
                                             int lane, int srank)
{
    constexpr int NCH = D / 8;
    constexpr int NT = SPLIT ? 128 : kLseWaves * 64;   // threads that move key tiles
    using Stg = std::conditional_t<KV8, StagerQ8<D, false, NT>, Stager<NCH, false, NT>>;
    const Stg stg(SPLIT ? (srank < 0 ? 0 : srank) : (int)threadIdx.x);
    const int n = it.n_rowtiles;
    int first = 0;
    for (int w = 0; w < wave; ++w)
        first += lse_rows(n, w);
    switch (lse_rows(n, wave)) {
    case 0: lse_body<D, 0, KV8, SPLIT>(a, it, pr, stg, lds_k, lds_kl, first, lane, srank); break;
    case 1: lse_body<D, 1, KV8, SPLIT>(a, it, pr, stg, lds_k, lds_kl, first, lane, srank); break;
    case 2: lse_body<D, 2, KV8, SPLIT>(a, it, pr, stg, lds_k, lds_kl, first, lane, srank); break;
    case 3: lse_body<D, 3, KV8, SPLIT>(a, it, pr, stg, lds_k, lds_kl, first, lane, srank); break;
    default: lse_body<D, 4, KV8, SPLIT>(a, it, pr, stg, lds_k, lds_kl, first, lane, srank); break;
    }
}

template <int D, bool KV8>
__global__ void __launch_bounds__(kLseWaves * 64, 1) attn_lse_kernel(const AttnArgs a)
{
    __shared__ __attribute__((aligned(16))) unsigned char lds_k[4][kTileK<D / 8>];
    __shared__ __attribute__((aligned(16))) unsigned char lds_kl[KV8 ? 4 : 1][KV8 ? kTileK<D / 8> : 16];

    const ItemDesc it = a.items[blockIdx.x];
    if (it.n_rowtiles == 0 || it.n_ktiles == 0)
        return;
    const ProbDesc pr = a.probs[it.prob];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    static_assert(kLseWaves == 8 && kLseMaxRowTilesPerWave == 4, "a body per row-tile count");
    if constexpr (!KV8) {
        const int r = it.n_rowtiles % 4;
        if (r >= 1) {
            // staging waves: the second waves of SIMDs 2 and 3 (r <= 2), or
            // both waves of SIMD 3 (r = 3)
            const int w0 = r <= 2 ? 6 : 3;
            const int srank = wave == w0 ? lane : wave == 7 ? 64 + lane : -1;
            lse_dispatch<D, KV8, true>(a, it, pr, lds_k, lds_kl, wave, lane, srank);
            return;
        }
    }
    lse_dispatch<D, KV8, false>(a, it, pr, lds_k, lds_kl, wave, lane, -1);
}

// The items of a plan whose blocks hold at most kLseWaves *
// kLseMaxRowTilesPerWave row tiles (the bf16 kernels' blocks: 4 * RT).
hipError_t launch_attn_lse(int d, bool kv8, const AttnArgs &args, int n_items, hipStream_t stream)
{
    if (n_items <= 0)
        return hipSuccess;
    const dim3 grid(n_items), block(kLseWaves * 64);
    if (d == 128) {
        if (kv8)
            hipLaunchKernelGGL((attn_lse_kernel<128, true>), grid, block, 0, stream, args);
        else
            hipLaunchKernelGGL((attn_lse_kernel<128, false>), grid, block, 0, stream, args);
    } else {
        if (kv8)
            hipLaunchKernelGGL((attn_lse_kernel<64, true>), grid, block, 0, stream, args);
        else
            hipLaunchKernelGGL((attn_lse_kernel<64, false>), grid, block, 0, stream, args);
    }
    return hipGetLastError();
}

// Output rows of split row blocks: each range's pass 2 wrote its fp32
// partial sum_i p_ji v_i over the range's keys (p already normalised by the
// block's full lse), so out_j is their sum, taken in range order (the same
// result on every run), rounded once to bf16. One workgroup per (split
// block, 16-row tile); a thread sums 4 columns of a row.
template <int D>
__global__ void __launch_bounds__(256) attn_out_combine_kernel(const CombineArgs a)
{
    constexpr int V4 = D / 4;   // float4 per row
    const OutCombItem ci = a.items[blockIdx.x];
    const ProbDesc pr = a.probs[ci.prob];
    const int G = a.G;
    const int packed_total = G * pr.rows;
    const gptr<const f32x4> src = as_global(reinterpret_cast<const f32x4 *>(a.opart + ci.opart));
    const size_t stride4 = (size_t)a.range_stride / 4;
#pragma unroll
    for (int e0 = 0; e0 < kRowTile * V4; e0 += 256) {
        const int e = e0 + threadIdx.x;
        const int lr = e / V4, c4 = e - (e / V4) * V4;
        const int r = ci.tile * kRowTile + lr;
        if (e >= kRowTile * V4 || r >= packed_total)
            continue;
        f32x4 acc = src[(size_t)lr * V4 + c4];
        for (int k = 1; k < ci.n_ranges; ++k) {
            const f32x4 v = src[k * stride4 + (size_t)lr * V4 + c4];
            acc[0] += v[0];
            acc[1] += v[1];
            acc[2] += v[2];
            acc[3] += v[3];
        }
        const int j = r / G;
        const int h = ci.kv_head * G + (r - j * G);
        const __bf16 b0 = (__bf16)acc[0], b1 = (__bf16)acc[1], b2 = (__bf16)acc[2], b3 = (__bf16)acc[3];
        const uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
        const uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, b2) | ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
        const gptr<uint16_t> orow = as_global(reinterpret_cast<uint16_t *>(pr.out)) + ((size_t)h * pr.rows + j) * D;
        *reinterpret_cast<gptr<u32x2>>(orow + 4 * c4) = u32x2{lo, hi};
    }
}

hipError_t launch_attn_out_combine(int d, const CombineArgs &args, int n_items, hipStream_t stream)
{
    if (n_items <= 0)
        return hipSuccess;
    if (d == 128)
        hipLaunchKernelGGL((attn_out_combine_kernel<128>), dim3(n_items), dim3(256), 0, stream, args);
    else
        hipLaunchKernelGGL((attn_out_combine_kernel<64>), dim3(n_items), dim3(256), 0, stream, args);
    return hipGetLastError();
}

}  // namespace crkv
