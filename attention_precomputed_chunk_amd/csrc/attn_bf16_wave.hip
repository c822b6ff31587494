// bf16 attention of query rows over a segment table of precomputed K/V
// chunks, with per-key impact partials, for gfx950 (CDNA4): the one-wave-per-
// SIMD kernel.
//
// What is computed (TurboRAG summary: K_combined = Concat(K^(1..m), K^(Q)) and
// the causal attention equation; CacheBlend summary: the Impact equation and
// the selective-recompute listing's softmax and column sum):
//   s_ji  = q_j . k_i / sqrt(d)      for keys at positions <= the row's
//   p_ji  = exp(s_ji - lse_j),  lse_j = log sum_i exp(s_ji)
//   out_j = sum_i p_ji v_i
//   imp_i = sum over heads and counted rows of p_ji
//
// Exact impact needs every row's final lse before any column sum, so each
// workgroup sweeps its keys twice: sweep 1 computes the row lse, sweep 2
// recomputes the scores, forms p in fp32, accumulates the impact column sums
// from the fp32 p, and runs P.V on the matrix cores with p rounded to bf16.
//
// The MFMA operand layout is described in attn_bf16_common.h.
//
// One wave per SIMD holds every role: Q fragments, the scores, the softmax and
// the O accumulators of its row tiles, so a KV head's rows fit in fewer
// workgroups than with the producer/consumer pairs of attn_bf16_pair.hip (up
// to 4 * 7 row tiles against 4 * 6), at the price of a wave that has to hide
// its own dependence latencies: sweep 2 is software-pipelined over the row
// tiles so the matrix cores and the vector ALU of the SIMD work at the same
// time (on the 32-layer GQA workload this took sweep 2 from about 3500 to 3000
// cycles per key tile; the same treatment made sweep 1, whose softmax chains
// the compiler already interleaves across row tiles, slower, so sweep 1 keeps
// the compiler's schedule). Each wave owns a compile-time number of
// 16-row tiles (no per-row-tile branches; padded rows are masked by an
// infinite lse), K/V tiles are staged through registers, and there is one
// barrier per 32-key tile.
//
// Work decomposition: one workgroup of 4 waves per (problem, KV head, block of
// 4 * RT row tiles). The rows of the G query heads sharing a KV head are
// packed as (query row j, head h) so one K/V tile in LDS serves the group.
#include <type_traits>

#include "attn_bf16_common.h"

namespace crkv {

// Who moves the key tiles into LDS and writes the impact partials: every
// wave its share (kSideShare), or, when the block's last wave holds at least
// kSideSlack fewer row tiles than the others, that wave alone (kSideAll)
// while the others only compute (kSideNone). The side work then runs in the
// last wave's slack instead of on every wave's critical path.
enum { kSideShare = 0, kSideNone = 1, kSideAll = 2 };
constexpr int kSideSlack = 2;

// One wave's part of a work item: RT row tiles per wave in the block (the
// stride of the waves' tile runs), RTW of them this wave's (RTW <= RT; the
// last wave of a partial block holds fewer).
template <int D, int RT, int RTW, int SIDE, bool CROSS, bool KV8, bool LSE_IN>
__device__ __forceinline__ void wave_body(const AttnArgs &a, const ItemDesc &it,
                                          unsigned char (*lds_k)[kTileK<D / 8>],
                                          unsigned char (*lds_v)[kTileV<D / 8>],
                                          unsigned char (*lds_kl)[KV8 ? kTileK<D / 8> : 16],
                                          float (*lds_imp)[kWaves][kKeyTile])
{
    static_assert(SIDE == kSideShare || (LSE_IN && !KV8), "side-work split: bf16, pass 1 on its own");
    static_assert(RTW >= 0 && RTW <= RT && (RTW > 0 || SIDE == kSideAll), "row tiles of the wave");
    constexpr int RTA = RTW > 0 ? RTW : 1;     // array extents
    constexpr int NT = kThreads;
    constexpr int NW = kWaves;
    constexpr int KS = D / 32;                 // MFMA k-steps along d
    constexpr int DT = D / 16;                 // output d tiles
    constexpr int NCH = D / 8;                 // 16-byte chunks per row
    static_assert(kKeyTile == 32, "tile geometry");
    // bf16 segments are staged as they are; 8-bit ones are widened on the way
    // (K into a bf16 hi/lo pair of tiles, V into one bf16 tile)
    using Stg1 = std::conditional_t<KV8, StagerQ8<D, false, NT>, Stager<NCH, false, NT>>;
    using Stg2 = std::conditional_t<KV8, StagerQ8<D, true, NT>,
                                    std::conditional_t<SIDE == kSideAll, Stager<NCH, true, 64>, Stager<NCH, true, NT>>>;
    constexpr bool STAGES = SIDE != kSideNone;   // this wave moves key tiles
    const Stg1 stg1(threadIdx.x);
    const Stg2 stg2(SIDE == kSideAll ? (int)(threadIdx.x & 63) : (int)threadIdx.x);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const ProbDesc pr = a.probs[it.prob];
    const int G = a.G;
    const float c = a.c_log2;
    const int packed_total = G * pr.rows;
    const int t0 = it.tile_begin + wave * RT;
    const int wave_min_pos = pr.pos0 + (t0 * kRowTile) / G;
    auto stage_load = [&](const auto &stg, TileSR kt) {
        if constexpr (KV8)
            return stg.load(kt, it.kv_head, a.H_kv);
        else
            return stg.load(kt, it.kv_head);
    };
    auto stage_store = [&](const auto &stg, const auto &st, int buf) {
        if constexpr (KV8)
            stg.store(st, lds_k[buf], lds_kl[buf], lds_v[buf]);
        else
            stg.store(st, lds_k[buf], lds_v[buf]);
    };

    int row_pos[RTA];
    bf16x8 qf[RTA][KS];
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
        const int r = (t0 + rt) * kRowTile + li;
        const bool valid = r < packed_total;
        const int j = r / G;
        const int h = it.kv_head * G + (r - j * G);
        row_pos[rt] = valid ? pr.pos0 + j : 0x3fffffff;
        const gptr<const u32x4> qrow = as_global(reinterpret_cast<const u32x4 *>(pr.Q)) + (size_t)(valid ? h * pr.rows + j : 0) * NCH;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const u32x4 q = valid ? qrow[4 * ks + lg] : u32x4{0u, 0u, 0u, 0u};
            qf[rt][ks] = __builtin_bit_cast(bf16x8, q);
        }
    }

    // Per-lane LDS byte offsets inside a tile.
    auto k_off = [&](int sub, int ks) { return k_frag_off<NCH>(li, lg, sub, ks); };
    auto v_off = [&](int dt, int r) { return v_frag_off<NCH>(li, lg, r, dt); };

    const int n_kt = it.n_ktiles;   // key tiles kt0 .. kt0 + n_kt - 1 of the problem's list
    const int kt0 = it.kt_begin;
    // ---------------------------------------------------------------- sweep 1: row lse
    float row_m[RTA], row_l[RTA];
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
        row_m[rt] = -INFINITY;
        row_l[rt] = 0.f;
    }
    auto sweep1_tile = [&](TileSR kt, int buf, auto mask_tag) {
        constexpr bool MASK = decltype(mask_tag)::value;
        bf16x8 kf[2][KS], kfl[KV8 ? 2 : 1][KS];
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                kf[sub][ks] = *reinterpret_cast<const bf16x8 *>(&lds_k[buf][k_off(sub, ks)]);
                if constexpr (KV8)
                    kfl[sub][ks] = *reinterpret_cast<const bf16x8 *>(&lds_kl[buf][k_off(sub, ks)]);
            }
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt) {
            f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f}, s1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[0][ks], qf[rt][ks], s0, 0, 0, 0);
                s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[1][ks], qf[rt][ks], s1, 0, 0, 0);
                if constexpr (KV8) {
                    s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfl[0][ks], qf[rt][ks], s0, 0, 0, 0);
                    s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfl[1][ks], qf[rt][ks], s1, 0, 0, 0);
                }
            }
            if constexpr (MASK) {
                const int lim = min(kt.n_valid - 1, row_pos[rt] - kt.key0);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (acc_key(lg, 0, e) > lim)
                        s0[e] = -INFINITY;
                    if (acc_key(lg, 1, e) > lim)
                        s1[e] = -INFINITY;
                }
            }
            const float tmax = fmaxf(fmaxf(fmaxf(row_m[rt], s0[0]), fmaxf(s0[1], s0[2])),
                                     fmaxf(fmaxf(s0[3], s1[0]), fmaxf(fmaxf(s1[1], s1[2]), s1[3])));
            const float mc = ((tmax == -INFINITY) ? 0.f : tmax) * c;
            float sum = exp2_hw(__builtin_fmaf(s0[0], c, -mc)) + exp2_hw(__builtin_fmaf(s1[0], c, -mc));
#pragma unroll
            for (int e = 1; e < 4; ++e)
                sum += exp2_hw(__builtin_fmaf(s0[e], c, -mc)) + exp2_hw(__builtin_fmaf(s1[e], c, -mc));
            row_l[rt] = __builtin_fmaf(row_l[rt], exp2_hw(__builtin_fmaf(row_m[rt], c, -mc)), sum);
            row_m[rt] = tmax;
        }
    };

    // Unmasked tile against the reference maxima; returns false, changing
    // nothing, when some row needs its maximum taken again (sweep1_tile then
    // redoes the tile exactly).
    auto sweep1_tile_ref = [&](int buf) -> bool {
        bf16x8 kf[2][KS], kfl[KV8 ? 2 : 1][KS];
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                kf[sub][ks] = *reinterpret_cast<const bf16x8 *>(&lds_k[buf][k_off(sub, ks)]);
                if constexpr (KV8)
                    kfl[sub][ks] = *reinterpret_cast<const bf16x8 *>(&lds_kl[buf][k_off(sub, ks)]);
            }
        float sum[RTA];
        bool big = false;
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt) {
            f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f}, s1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[0][ks], qf[rt][ks], s0, 0, 0, 0);
                s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[1][ks], qf[rt][ks], s1, 0, 0, 0);
                if constexpr (KV8) {
                    s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfl[0][ks], qf[rt][ks], s0, 0, 0, 0);
                    s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfl[1][ks], qf[rt][ks], s1, 0, 0, 0);
                }
            }
            const float mc = row_m[rt] * c;
            float e[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                e[i] = exp2_hw(__builtin_fmaf(s0[i], c, -mc));
                e[4 + i] = exp2_hw(__builtin_fmaf(s1[i], c, -mc));
            }
            sum[rt] = ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
            big |= sum[rt] > kLseRescaleBound;
        }
        if (__builtin_amdgcn_ballot_w64(big))
            return false;
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt)
            row_l[rt] += sum[rt];
        return true;
    };

    // Descriptors are loaded two tiles ahead of use and data one tile ahead;
    // a descriptor reaches scalar registers one iteration after its load.
    auto desc = [&](int tt) { return load_tile(pr.tiles, kt0 + min(tt, n_kt - 1), lane); };
    if (!LSE_IN && n_kt > 0) {
        TileSR cur = to_sr(desc(0));
        uint32_t nraw = desc(1);
        stage_store(stg1, stage_load(stg1, cur), 0);
        __syncthreads();
        for (int tt = 0; tt < n_kt; ++tt) {
            const int buf = tt & 1;
            const bool more = tt + 1 < n_kt;
            const TileSR nxt = to_sr(nraw);
            nraw = desc(tt + 2);
            decltype(stage_load(stg1, nxt)) st;
            if (more)
                st = stage_load(stg1, nxt);
            const bool need_mask = (cur.n_valid < kKeyTile) || (cur.key0 + cur.n_valid - 1 > wave_min_pos);
            if (need_mask)
                sweep1_tile(cur, buf, std::true_type{});
            else if (!sweep1_tile_ref(buf))
                sweep1_tile(cur, buf, std::false_type{});
            if (more)
                stage_store(stg1, st, buf ^ 1);
            __syncthreads();
            cur = nxt;
        }
    }

    // Combine the four lane groups of each row into its log2-domain lse;
    // padded rows get +inf so every weight they would produce is 0. With
    // LSE_IN pass 1 ran as attn_lse_kernel, one state per range of the block
    // (written for the block's real row tiles only).
    float lse2[RTA];
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
        if constexpr (LSE_IN) {
            lse2[rt] = (row_pos[rt] < 0x3fffffff) ? merged_lse(a, it, (wave * RT + rt) * kRowTile + li, c) : INFINITY;
        } else {
            float m = row_m[rt], l = row_l[rt];
            merge_state(m, l, __shfl_xor(m, 16), __shfl_xor(l, 16), c);
            merge_state(m, l, __shfl_xor(m, 32), __shfl_xor(l, 32), c);
            lse2[rt] = (row_pos[rt] < 0x3fffffff) ? m * c + __log2f(l) : INFINITY;
        }
    }

    // ---------------------------------------------------------------- sweep 2: P.V and impact
    f32x4 o[RTA][DT];
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
            o[rt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};

    const gptr<float> partial = as_global(pr.partial) + (size_t)it.slot * pr.n_keys;
    // A tile's partial: its waves' sums are read from LDS at the top of the
    // next iteration (flush_read) and added and written after that
    // iteration's arithmetic (flush_write), so the LDS latency hides under it.
    auto flush_mine = [&](int tt) { return SIDE == kSideAll || (SIDE == kSideShare && wave == tt % NW); };
    auto flush_read = [&](int tt, int buf, float (&fv)[NW]) {
        if (flush_mine(tt) && lane < kKeyTile) {
#pragma unroll
            for (int w = 0; w < NW; ++w)
                fv[w] = lds_imp[buf][w][lane];
        }
    };
    auto flush_write = [&](int tt, TileSR kt, const float (&fv)[NW]) {
        if (flush_mine(tt) && lane < kt.n_valid) {
            float sum = fv[0];
#pragma unroll
            for (int w = 1; w < NW; ++w)
                sum += fv[w];
            partial[kt.key0 + lane] = sum;
        }
    };
    // Tiles that need the causal or ragged-tail mask.
    auto sweep2_tile = [&](TileSR kt, int buf, auto mask_tag) {
        constexpr bool MASK = decltype(mask_tag)::value;
        bf16x8 kf[2][KS], kfl[KV8 ? 2 : 1][KS], vf[DT];
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                kf[sub][ks] = *reinterpret_cast<const bf16x8 *>(&lds_k[buf][k_off(sub, ks)]);
                if constexpr (KV8)
                    kfl[sub][ks] = *reinterpret_cast<const bf16x8 *>(&lds_kl[buf][k_off(sub, ks)]);
            }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4 *)(&lds_v[buf][v_off(dt, 0)]));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4 *)(&lds_v[buf][v_off(dt, 1)]));
            vf[dt] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
        float imp[8];
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt) {
            f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f}, s1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[0][ks], qf[rt][ks], s0, 0, 0, 0);
                s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[1][ks], qf[rt][ks], s1, 0, 0, 0);
                if constexpr (KV8) {
                    s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfl[0][ks], qf[rt][ks], s0, 0, 0, 0);
                    s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfl[1][ks], qf[rt][ks], s1, 0, 0, 0);
                }
            }
            if constexpr (MASK) {
                const int lim = min(kt.n_valid - 1, row_pos[rt] - kt.key0);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (acc_key(lg, 0, e) > lim)
                        s0[e] = -INFINITY;
                    if (acc_key(lg, 1, e) > lim)
                        s1[e] = -INFINITY;
                }
            }
            float p[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                p[e] = exp2_hw(__builtin_fmaf(s0[e], c, -lse2[rt]));
                p[4 + e] = exp2_hw(__builtin_fmaf(s1[e], c, -lse2[rt]));
            }
            if constexpr (CROSS) {
                // rows inside the tile's own segment do not count
                const float w = (row_pos[rt] >= kt.seg_lo && row_pos[rt] < kt.seg_lo + kt.seg_len) ? 0.f : 1.f;
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    imp[i] = rt == 0 ? p[i] * w : __builtin_fmaf(p[i], w, imp[i]);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    imp[i] = rt == 0 ? p[i] : imp[i] + p[i];
            }
            bf16x8 pb;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                pb[i] = (__bf16)p[i];
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                o[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[dt], pb, o[rt][dt], 0, 0, 0);
        }
        float i0, i1;
        row16_sum8(imp, li, i0, i1);
        if ((li & 3) == 0)
            *reinterpret_cast<float2 *>(&lds_imp[buf][wave][imp_key(li, lg)]) = make_float2(i0, i1);
    };

    // Unmasked tiles, software-pipelined over the row tiles: stage rt issues
    // the score MFMAs of row tile rt + 1 and the P.V MFMAs of row tile rt - 1
    // between the vector instructions that turn row tile rt's scores into p
    // (exp, impact sums, bf16 rounding). Every stage is a scheduling region.
    auto sweep2_tile_pipe = [&](TileSR kt, int buf) {
        bf16x8 kf[2][KS], kfl[KV8 ? 2 : 1][KS], vf[DT];
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                kf[sub][ks] = *reinterpret_cast<const bf16x8 *>(&lds_k[buf][k_off(sub, ks)]);
                if constexpr (KV8)
                    kfl[sub][ks] = *reinterpret_cast<const bf16x8 *>(&lds_kl[buf][k_off(sub, ks)]);
            }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4 *)(&lds_v[buf][v_off(dt, 0)]));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4 *)(&lds_v[buf][v_off(dt, 1)]));
            vf[dt] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
        float imp[8];
        f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f}, s1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[0][ks], qf[0][ks], s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[1][ks], qf[0][ks], s1, 0, 0, 0);
            if constexpr (KV8) {
                s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfl[0][ks], qf[0][ks], s0, 0, 0, 0);
                s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfl[1][ks], qf[0][ks], s1, 0, 0, 0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 pprev;
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt) {
            f32x4 n0 = f32x4{0.f, 0.f, 0.f, 0.f}, n1 = f32x4{0.f, 0.f, 0.f, 0.f};
            if (rt + 1 < RTW) {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    n0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[0][ks], qf[rt + 1][ks], n0, 0, 0, 0);
                    n1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[1][ks], qf[rt + 1][ks], n1, 0, 0, 0);
                    if constexpr (KV8) {
                        n0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfl[0][ks], qf[rt + 1][ks], n0, 0, 0, 0);
                        n1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfl[1][ks], qf[rt + 1][ks], n1, 0, 0, 0);
                    }
                }
            }
            if (rt > 0) {
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
                    o[rt - 1][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[dt], pprev, o[rt - 1][dt], 0, 0, 0);
            }
            float p[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                p[e] = exp2_hw(__builtin_fmaf(s0[e], c, -lse2[rt]));
                p[4 + e] = exp2_hw(__builtin_fmaf(s1[e], c, -lse2[rt]));
            }
            if constexpr (CROSS) {
                const float w = (row_pos[rt] >= kt.seg_lo && row_pos[rt] < kt.seg_lo + kt.seg_len) ? 0.f : 1.f;
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    imp[i] = rt == 0 ? p[i] * w : __builtin_fmaf(p[i], w, imp[i]);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    imp[i] = rt == 0 ? p[i] : imp[i] + p[i];
            }
#pragma unroll
            for (int i = 0; i < 8; ++i)
                pprev[i] = (__bf16)p[i];
            constexpr int QK = (KV8 ? 4 : 2) * KS;   // score MFMAs of a row tile
            constexpr int n_mfma_max = QK + DT;
            const int n_mfma = (rt + 1 < RTW ? QK : 0) + (rt > 0 ? DT : 0);
#pragma unroll
            for (int i = 0; i < n_mfma_max; ++i) {
                if (i < n_mfma) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x402, 2, 0);   // VALU and transcendental
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            s0 = n0;
            s1 = n1;
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
            o[RTA - 1][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[dt], pprev, o[RTA - 1][dt], 0, 0, 0);
        float i0, i1;
        row16_sum8(imp, li, i0, i1);
        if ((li & 3) == 0)
            *reinterpret_cast<float2 *>(&lds_imp[buf][wave][imp_key(li, lg)]) = make_float2(i0, i1);
    };

    if (n_kt > 0) {
        TileSR cur = to_sr(desc(0)), prev = cur;
        uint32_t nraw = desc(1);
        if constexpr (STAGES)
            stage_store(stg2, stage_load(stg2, cur), 0);
        __syncthreads();
        for (int tt = 0; tt < n_kt; ++tt) {
            const int buf = tt & 1;
            const bool more = tt + 1 < n_kt;
            const TileSR nxt = to_sr(nraw);
            nraw = desc(tt + 2);
            decltype(stage_load(stg2, nxt)) st;
            if (STAGES && more)
                st = stage_load(stg2, nxt);
            float fv[NW];
            if (tt > 0)
                flush_read(tt - 1, buf ^ 1, fv);
            if constexpr (RTW > 0) {
                const bool need_mask = (cur.n_valid < kKeyTile) || (cur.key0 + cur.n_valid - 1 > wave_min_pos);
                if (need_mask)
                    sweep2_tile(cur, buf, std::true_type{});
                else
                    sweep2_tile_pipe(cur, buf);
            } else {
                // no rows: this wave's impact sums of the tile are zero
                if ((lane & 15) == 0)
                    for (int i = 0; i < 8; ++i)
                        lds_imp[buf][wave][8 * (lane >> 4) + i] = 0.f;
            }
            if (tt > 0)
                flush_write(tt - 1, prev, fv);
            if (STAGES && more)
                stage_store(stg2, st, buf ^ 1);
            __syncthreads();
            prev = cur;
            cur = nxt;
        }
        float fv[NW];
        flush_read(n_kt - 1, (n_kt - 1) & 1, fv);
        flush_write(n_kt - 1, prev, fv);
    }

    // ---------------------------------------------------------------- epilogue: out rows
    // (a block split into key ranges writes this range's fp32 partial rows;
    // attn_out_combine_kernel sums them)
    if (LSE_IN && it.n_ranges > 1) {
        const gptr<f32x4> part = as_global(reinterpret_cast<f32x4 *>(a.opart + it.opart)) +
                                 (size_t)it.range * (a.cap_rows * D / 4);
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt) {
            const int local = (wave * RT + rt) * kRowTile + li;
            if ((t0 + rt) * kRowTile + li >= packed_total)
                continue;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                part[(size_t)local * (D / 4) + 4 * dt + lg] = o[rt][dt];
        }
        return;
    }
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
        const int r = (t0 + rt) * kRowTile + li;
        if (r >= packed_total)
            continue;
        const int j = r / G;
        const int h = it.kv_head * G + (r - j * G);
        const gptr<uint16_t> orow = as_global(reinterpret_cast<uint16_t *>(pr.out)) + ((size_t)h * pr.rows + j) * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const __bf16 b0 = (__bf16)o[rt][dt][0], b1 = (__bf16)o[rt][dt][1];
            const __bf16 b2 = (__bf16)o[rt][dt][2], b3 = (__bf16)o[rt][dt][3];
            const uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, b0) |
                                ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
            const uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, b2) |
                                ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
            *reinterpret_cast<gptr<u32x2>>(orow + 16 * dt + 4 * lg) = u32x2{lo, hi};
        }
    }
}


template <int D, int RT, bool CROSS, bool KV8, bool LSE_IN>
__global__ void __launch_bounds__(kThreads, 1) attn_bf16_wave_kernel(const AttnArgs a)
{
    __shared__ __attribute__((aligned(16))) unsigned char lds_k[2][kTileK<D / 8>];
    __shared__ __attribute__((aligned(16))) unsigned char lds_v[2][kTileV<D / 8>];
    __shared__ __attribute__((aligned(16))) unsigned char lds_kl[KV8 ? 2 : 1][KV8 ? kTileK<D / 8> : 16];   // K lo (8-bit)
    __shared__ float lds_imp[2][kWaves][kKeyTile];
    const ItemDesc it = a.items[blockIdx.x];
    if (it.n_rowtiles == 0)
        return;
    if constexpr (LSE_IN && !KV8 && RT == 7) {
        // the last wave's row tiles; with kSideSlack or more fewer than RT it
        // takes over every wave's staging and impact flushes
        const int last = it.n_rowtiles - (kWaves - 1) * RT;
        if (last >= 0 && last <= RT - kSideSlack) {
            const int wave = threadIdx.x >> 6;
            if (wave < kWaves - 1) {
                wave_body<D, RT, RT, kSideNone, CROSS, KV8, LSE_IN>(a, it, lds_k, lds_v, lds_kl, lds_imp);
                return;
            }
            switch (last) {
            case 0: wave_body<D, RT, 0, kSideAll, CROSS, KV8, LSE_IN>(a, it, lds_k, lds_v, lds_kl, lds_imp); break;
            case 1: wave_body<D, RT, 1, kSideAll, CROSS, KV8, LSE_IN>(a, it, lds_k, lds_v, lds_kl, lds_imp); break;
            case 2: wave_body<D, RT, 2, kSideAll, CROSS, KV8, LSE_IN>(a, it, lds_k, lds_v, lds_kl, lds_imp); break;
            case 3: wave_body<D, RT, 3, kSideAll, CROSS, KV8, LSE_IN>(a, it, lds_k, lds_v, lds_kl, lds_imp); break;
            case 4: wave_body<D, RT, 4, kSideAll, CROSS, KV8, LSE_IN>(a, it, lds_k, lds_v, lds_kl, lds_imp); break;
            default: wave_body<D, RT, 5, kSideAll, CROSS, KV8, LSE_IN>(a, it, lds_k, lds_v, lds_kl, lds_imp); break;
            }
            return;
        }
    }
    wave_body<D, RT, RT, kSideShare, CROSS, KV8, LSE_IN>(a, it, lds_k, lds_v, lds_kl, lds_imp);
}

template <int D, int RT, bool KV8, bool LSE_IN>
static void launch_wave_rt2(const AttnArgs &args, int n_items, hipStream_t stream)
{
    if constexpr (RT <= kWaveMaxRowTilesCross) {
        if (args.cross) {
            hipLaunchKernelGGL((attn_bf16_wave_kernel<D, RT, true, KV8, LSE_IN>), dim3(n_items), dim3(kThreads), 0,
                               stream, args);
            return;
        }
    }
    hipLaunchKernelGGL((attn_bf16_wave_kernel<D, RT, false, KV8, LSE_IN>), dim3(n_items), dim3(kThreads), 0, stream,
                       args);
}

// args.state non-null: pass 1 already ran (attn_lse_kernel) and pass 2 reads it.
template <int D, int RT, bool KV8>
static void launch_wave_rt(const AttnArgs &args, int n_items, hipStream_t stream)
{
    if (args.state)
        launch_wave_rt2<D, RT, KV8, true>(args, n_items, stream);
    else
        launch_wave_rt2<D, RT, KV8, false>(args, n_items, stream);
}

hipError_t launch_attn_bf16_wave(int d, int rt, const AttnArgs &args, int n_items, hipStream_t stream)
{
    if (n_items <= 0)
        return hipSuccess;
    if (args.cross && rt > kWaveMaxRowTilesCross)
        return hipErrorInvalidValue;   // no such build; the planner never asks for it
    if (d == 128) {
        switch (rt) {
        case 1: launch_wave_rt<128, 1, false>(args, n_items, stream); break;
        case 2: launch_wave_rt<128, 2, false>(args, n_items, stream); break;
        case 4: launch_wave_rt<128, 4, false>(args, n_items, stream); break;
        case 5: launch_wave_rt<128, 5, false>(args, n_items, stream); break;
        case 7: launch_wave_rt<128, 7, false>(args, n_items, stream); break;
        default: return hipErrorInvalidValue;   // no such build; the planner never asks for it
        }
    } else {
        switch (rt) {
        case 1: launch_wave_rt<64, 1, false>(args, n_items, stream); break;
        case 2: launch_wave_rt<64, 2, false>(args, n_items, stream); break;
        case 4: launch_wave_rt<64, 4, false>(args, n_items, stream); break;
        case 5: launch_wave_rt<64, 5, false>(args, n_items, stream); break;
        case 7: launch_wave_rt<64, 7, false>(args, n_items, stream); break;
        default: return hipErrorInvalidValue;
        }
    }
    return hipGetLastError();
}

// Key tiles in the 8-bit format: the same kernel with K widened into a bf16
// hi/lo pair and V into bf16 while staging (row tiles per wave: 4 or 5).
hipError_t launch_attn_q8(int d, int rt, const AttnArgs &args, int n_items, hipStream_t stream)
{
    if (n_items <= 0)
        return hipSuccess;
    if (rt != 4 && rt != 5)
        return hipErrorInvalidValue;   // no such build; the planner never asks for it
    if (d == 128) {
        if (rt == 5)
            launch_wave_rt<128, 5, true>(args, n_items, stream);
        else
            launch_wave_rt<128, 4, true>(args, n_items, stream);
    } else {
        if (rt == 5)
            launch_wave_rt<64, 5, true>(args, n_items, stream);
        else
            launch_wave_rt<64, 4, true>(args, n_items, stream);
    }
    return hipGetLastError();
}

}  // namespace crkv
