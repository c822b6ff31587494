// bf16 attention of query rows over a segment table of precomputed K/V
// chunks, with per-key impact partials, for gfx950 (CDNA4): the
// producer/consumer wave-pair kernel.
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
// Waves and SIMDs. A wave issues in order and at most one instruction every
// few cycles, so a lone wave per SIMD leaves the matrix core idle while it
// works through the softmax and cannot hide the latency of its own
// dependences. Two waves per SIMD overlap one's vector work with the other's
// matrix work, but cannot each hold Q, K and V fragments and a d = 128 output
// accumulator in 256 registers. The workgroup therefore has 8 waves (waves w
// and w + 4 share a SIMD) with roles:
//   * sweep 1: every wave takes RT/2 row tiles and computes their lse, two
//     key tiles per barrier;
//   * sweep 2: wave p < 4 (producer) holds Q of RT row tiles, computes S and
//     p and the impact column sums, and writes P^T fragments (bf16) to LDS;
//     wave p + 4 (consumer) holds the O accumulators of the same rows and
//     runs P.V on the key tile the producer finished one step earlier.
// Each role runs its own loop, so the register allocator never holds Q and O
// at once; both loops meet the same barriers (one per step). LDS holds K
// twice (tile being scored, tile being staged), V three times (tile in P.V,
// tile being scored, tile being staged) and P^T twice.
//
// Work decomposition: one workgroup per (problem, KV head, block of 4 * RT row
// tiles). The rows of the G query heads sharing a KV head are packed as
// (query row j, head h) so one K/V tile in LDS serves the group.
#include <type_traits>

#include "attn_bf16_common.h"

namespace crkv {


template <int D, int RT, bool CROSS, bool LSE_IN>
__global__ void __launch_bounds__(kWsThreads) attn_bf16_pair_kernel(const AttnArgs a)
{
    constexpr int RT1 = RT / 2;                // row tiles per wave in sweep 1
    constexpr int KS = D / 32;                 // MFMA k-steps along d
    constexpr int DT = D / 16;                 // output d tiles
    constexpr int NCH = D / 8;                 // 16-byte chunks per row
    static_assert(kKeyTile == 32 && RT % 2 == 0, "tile geometry");

    // Sweep 1 stages K tiles into both arrays (a V tile is the larger).
    __shared__ __attribute__((aligned(16))) unsigned char lds_k[2][kTileK<NCH>];
    __shared__ __attribute__((aligned(16))) unsigned char lds_v[3][kTileV<NCH>];
    __shared__ __attribute__((aligned(16))) bf16x8 lds_p[2][kWaves][RT][64];
    __shared__ __attribute__((aligned(16))) float lds_imp[2][kWaves][kKeyTile];
    __shared__ float lds_lse[LSE_IN ? 1 : kWaves * RT * kRowTile];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 15, lg = lane >> 4;
    const ItemDesc it = a.items[blockIdx.x];
    if (it.n_rowtiles == 0)
        return;
    const ProbDesc pr = a.probs[it.prob];
    const int G = a.G;
    const float c = a.c_log2;
    const int n_kt = it.n_ktiles;   // key tiles kt0 .. kt0 + n_kt - 1 of the problem's list
    const int kt0 = it.kt_begin;
    if (n_kt == 0)
        return;

    // Per-lane LDS byte offsets inside a tile.
    auto k_off = [&](int sub, int ks) { return k_frag_off<NCH>(li, lg, sub, ks); };
    auto v_off = [&](int dt, int r) { return v_frag_off<NCH>(li, lg, r, dt); };
    auto desc = [&](int tt) { return load_tile(pr.tiles, kt0 + min(tt, n_kt - 1), lane); };
    auto min_pos = [&](int t0) { return pr.pos0 + (t0 * kRowTile) / G; };

    // ---------------------------------------------------------------- sweep 1: row lse (all waves)
    // (with LSE_IN pass 1 ran as attn_lse_kernel: one state per key range)
    if constexpr (!LSE_IN) {
        const int t0 = it.tile_begin + wave * RT1;
        const int wave_min_pos = min_pos(t0);
        bf16x8 qf[RT1][KS];
        int row_pos[RT1];
        float row_m[RT1], row_l[RT1];
#pragma unroll
        for (int rt = 0; rt < RT1; ++rt) {
            load_q_rows<KS>(pr, it, G, t0 + rt, li, lg, qf[rt], row_pos[rt]);
            row_m[rt] = -INFINITY;
            row_l[rt] = 0.f;
        }
        auto tile = [&](TileSR kt, const unsigned char *kb, auto mask_tag) {
            constexpr bool MASK = decltype(mask_tag)::value;
            bf16x8 kf[2][KS];
#pragma unroll
            for (int sub = 0; sub < 2; ++sub)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    kf[sub][ks] = *reinterpret_cast<const bf16x8 *>(kb + k_off(sub, ks));
#pragma unroll
            for (int rt = 0; rt < RT1; ++rt) {
                Spair sc = scores<KS>(kf, qf[rt]);
                if constexpr (MASK)
                    mask_scores(sc, min(kt.n_valid - 1, row_pos[rt] - kt.key0), lg);
                const f32x4 s0 = sc.s0, s1 = sc.s1;
                const float tmax = fmaxf(fmaxf(fmaxf(row_m[rt], s0[0]), fmaxf(s0[1], s0[2])),
                                         fmaxf(fmaxf(s0[3], s1[0]), fmaxf(fmaxf(s1[1], s1[2]), s1[3])));
                const float mc = ((tmax == -INFINITY) ? 0.f : tmax) * c;
                float sum = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sum += exp2_hw(__builtin_fmaf(s0[e], c, -mc)) + exp2_hw(__builtin_fmaf(s1[e], c, -mc));
                row_l[rt] = __builtin_fmaf(row_l[rt], exp2_hw(__builtin_fmaf(row_m[rt], c, -mc)), sum);
                row_m[rt] = tmax;
            }
        };
        auto run_tile = [&](TileSR kt, const unsigned char *kb) {
            if ((kt.n_valid < kKeyTile) || (kt.key0 + kt.n_valid - 1 > wave_min_pos))
                tile(kt, kb, std::true_type{});
            else
                tile(kt, kb, std::false_type{});
        };
        // Two key tiles per barrier. Step g scores tiles 2g and 2g + 1 from
        // the buffers of its parity (sweep 2's lds_k[0..1] for even g, its
        // lds_v[0..1] for odd g) while tiles 2g + 2 and 2g + 3 are loaded and
        // then stored into the other parity's buffers.
        auto sbuf = [&](int g, int j) -> unsigned char * { return (g & 1) ? lds_v[j] : lds_k[j]; };
        const Stager<NCH, false, kWsThreads> stg(tid);
        TileSR c0 = to_sr(desc(0)), c1 = to_sr(desc(1));
        stg.store(stg.load(c0, it.kv_head), sbuf(0, 0), nullptr);
        if (n_kt > 1)
            stg.store(stg.load(c1, it.kv_head), sbuf(0, 1), nullptr);
        uint32_t raw0 = desc(2), raw1 = desc(3);
        __syncthreads();
        const int n_steps = (n_kt + 1) / 2;
        for (int g = 0; g < n_steps; ++g) {
            const int ta = 2 * g + 2, tb = 2 * g + 3;   // tiles loaded during this step
            const TileSR s0 = to_sr(raw0), s1 = to_sr(raw1);
            raw0 = desc(ta + 2);
            raw1 = desc(tb + 2);
            Staged<NCH, false, kWsThreads> sa, sb;
            if (ta < n_kt)
                sa = stg.load(s0, it.kv_head);
            if (tb < n_kt)
                sb = stg.load(s1, it.kv_head);
            run_tile(c0, sbuf(g, 0));
            if (2 * g + 1 < n_kt)
                run_tile(c1, sbuf(g, 1));
            if (ta < n_kt)
                stg.store(sa, sbuf(g + 1, 0), nullptr);
            if (tb < n_kt)
                stg.store(sb, sbuf(g + 1, 1), nullptr);
            __syncthreads();
            c0 = s0;
            c1 = s1;
        }
        // Combine the four lane groups of each row into its log2-domain lse;
        // padded rows get +inf so every weight they would produce is 0.
#pragma unroll
        for (int rt = 0; rt < RT1; ++rt) {
            float m = row_m[rt], l = row_l[rt];
            merge_state(m, l, __shfl_xor(m, 16), __shfl_xor(l, 16), c);
            merge_state(m, l, __shfl_xor(m, 32), __shfl_xor(l, 32), c);
            if (lg == 0)
                lds_lse[(wave * RT1 + rt) * kRowTile + li] =
                    (row_pos[rt] < 0x3fffffff) ? m * c + __log2f(l) : INFINITY;
        }
    }

    // ---------------------------------------------------------------- sweep 2
    // Step s (0 <= s <= n_kt): the producers score key tile s from lds_k[s & 1]
    // and write its P^T to lds_p[s & 1]; the consumers run P.V of tile s - 1
    // from lds_p[(s - 1) & 1] and lds_v[(s - 1) % 3] and flush its impact;
    // tile s + 1 is loaded from global memory and stored into
    // lds_k[(s + 1) & 1] (by the producers) and lds_v[(s + 1) % 3] (by the
    // consumers, which have slack: the producers' scores, exponentials and
    // impact sums are the critical path). Every read of a buffer ends
    // before the barrier after which it is refilled.
    constexpr int NTP = kWaves * 64;
    const Stager<NCH, false, NTP> stgk(tid & (NTP - 1));   // K of a tile over one role's threads
    {
        const TileSR t = to_sr(desc(0));
        if (wave < kWaves)
            stgk.store(stgk.load(t, it.kv_head), lds_k[0], nullptr);
        else
            stgk.store_v(stgk.load_v(t, it.kv_head), lds_v[0]);
    }
    __syncthreads();   // also publishes lds_lse

    const int pair = wave & (kWaves - 1);
    const int t0 = it.tile_begin + pair * RT;
    if (wave < kWaves) {
        // ------------------------------------------------------------ producer
        const int wave_min_pos = min_pos(t0);
        bf16x8 qf[RT][KS];
        int row_pos[RT];
        float lse2[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            load_q_rows<KS>(pr, it, G, t0 + rt, li, lg, qf[rt], row_pos[rt]);
            if constexpr (LSE_IN)
                lse2[rt] = (row_pos[rt] < 0x3fffffff) ? merged_lse(a, it, (pair * RT + rt) * kRowTile + li, c)
                                                      : INFINITY;
            else
                lse2[rt] = lds_lse[(pair * RT + rt) * kRowTile + li];
        }
        auto tile = [&](TileSR kt, int buf, auto mask_tag) {
            constexpr bool MASK = decltype(mask_tag)::value;
            bf16x8 kf[2][KS];
#pragma unroll
            for (int sub = 0; sub < 2; ++sub)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    kf[sub][ks] = *reinterpret_cast<const bf16x8 *>(&lds_k[buf][k_off(sub, ks)]);
            float imp[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                imp[i] = 0.f;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                Spair sc = scores<KS>(kf, qf[rt]);
                if constexpr (MASK)
                    mask_scores(sc, min(kt.n_valid - 1, row_pos[rt] - kt.key0), lg);
                float p[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    p[e] = exp2_hw(__builtin_fmaf(sc.s0[e], c, -lse2[rt]));
                    p[4 + e] = exp2_hw(__builtin_fmaf(sc.s1[e], c, -lse2[rt]));
                }
                if constexpr (CROSS) {
                    // rows inside the tile's own segment do not count
                    const float w =
                        (row_pos[rt] >= kt.seg_lo && row_pos[rt] < kt.seg_lo + kt.seg_len) ? 0.f : 1.f;
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        imp[i] = __builtin_fmaf(p[i], w, imp[i]);
                } else {
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        imp[i] += p[i];
                }
                bf16x8 pb;
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    pb[i] = (__bf16)p[i];
                lds_p[buf][pair][rt][lane] = pb;
            }
            float i0, i1;
            row16_sum8(imp, li, i0, i1);
            if ((li & 3) == 0)
                *reinterpret_cast<float2 *>(&lds_imp[buf][pair][imp_key(li, lg)]) = make_float2(i0, i1);
        };
        TileSR cur = to_sr(desc(0));
        uint32_t craw = desc(1);
        for (int s = 0; s <= n_kt; ++s) {
            const TileSR nxt = to_sr(craw);
            craw = desc(s + 2);
            Staged<NCH, false, NTP> st;
            if (s + 1 < n_kt)
                st = stgk.load(nxt, it.kv_head);
            if (s < n_kt) {
                if ((cur.n_valid < kKeyTile) || (cur.key0 + cur.n_valid - 1 > wave_min_pos))
                    tile(cur, s & 1, std::true_type{});
                else
                    tile(cur, s & 1, std::false_type{});
            }
            if (s + 1 < n_kt)
                stgk.store(st, lds_k[(s + 1) & 1], nullptr);
            __syncthreads();
            cur = nxt;
        }
    } else {
        // ------------------------------------------------------------ consumer
        f32x4 o[RT][DT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                o[rt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        const gptr<float> partial = as_global(pr.partial) + (size_t)it.slot * pr.n_keys;
        TileSR cur = to_sr(desc(0)), prev = cur;
        uint32_t nraw = desc(1);
        int vb = 1;   // lds_v slot of tile s + 1; tile s - 1 sits in the next slot (mod 3)
        for (int s = 0; s <= n_kt; ++s) {
            const TileSR nxt = to_sr(nraw);
            nraw = desc(s + 2);
            Staged<NCH, false, NTP> st;
            if (s + 1 < n_kt)
                st = stgk.load_v(nxt, it.kv_head);
            if (s > 0) {
                const int pbuf = (s - 1) & 1;
                const int vprev = vb == 2 ? 0 : vb + 1;
                // impact of tile s - 1: one consumer adds the four producers' column sums
                if (pair == ((s - 1) & (kWaves - 1)) && lane < prev.n_valid)
                    partial[prev.key0 + lane] = lds_imp[pbuf][0][lane] + lds_imp[pbuf][1][lane] +
                                                lds_imp[pbuf][2][lane] + lds_imp[pbuf][3][lane];
                bf16x8 pb[RT];
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
                    pb[rt] = lds_p[pbuf][pair][rt][lane];
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
                    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_i16x4 *)(&lds_v[vprev][v_off(dt, 0)]));
                    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_i16x4 *)(&lds_v[vprev][v_off(dt, 1)]));
                    const bf16x8 vf =
                        __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt)
                        o[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb[rt], o[rt][dt], 0, 0, 0);
                }
            }
            if (s + 1 < n_kt)
                stgk.store_v(st, lds_v[vb]);
            __syncthreads();
            prev = cur;
            cur = nxt;
            vb = vb == 2 ? 0 : vb + 1;
        }

        // ------------------------------------------------------------ epilogue: out rows
        // (a block split into key ranges writes this range's fp32 partial
        // rows; attn_out_combine_kernel sums them)
        const int packed_total = G * pr.rows;
        if (LSE_IN && it.n_ranges > 1) {
            const gptr<f32x4> part = as_global(reinterpret_cast<f32x4 *>(a.opart + it.opart)) +
                                     (size_t)it.range * (a.cap_rows * D / 4);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const int local = (pair * RT + rt) * kRowTile + li;
                if ((t0 + rt) * kRowTile + li >= packed_total)
                    continue;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
                    part[(size_t)local * (D / 4) + 4 * dt + lg] = o[rt][dt];
            }
            return;
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const int r = (t0 + rt) * kRowTile + li;
            if (r >= packed_total)
                continue;
            const int j = r / G;
            const int h = it.kv_head * G + (r - j * G);
            const gptr<uint16_t> orow =
                as_global(reinterpret_cast<uint16_t *>(pr.out)) + ((size_t)h * pr.rows + j) * D;
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
}

// args.state non-null: pass 1 already ran (attn_lse_kernel) and sweep 1 is skipped.
template <int D, int RT, bool LSE_IN>
static void launch_pair_rt2(const AttnArgs &args, int n_items, hipStream_t stream)
{
    if (args.cross)
        hipLaunchKernelGGL((attn_bf16_pair_kernel<D, RT, true, LSE_IN>), dim3(n_items), dim3(kWsThreads), 0, stream,
                           args);
    else
        hipLaunchKernelGGL((attn_bf16_pair_kernel<D, RT, false, LSE_IN>), dim3(n_items), dim3(kWsThreads), 0, stream,
                           args);
}

template <int D, int RT>
static void launch_pair_rt(const AttnArgs &args, int n_items, hipStream_t stream)
{
    if (args.state)
        launch_pair_rt2<D, RT, true>(args, n_items, stream);
    else
        launch_pair_rt2<D, RT, false>(args, n_items, stream);
}

template <int D>
static hipError_t launch_pair_d(int rt, const AttnArgs &args, int n_items, hipStream_t stream)
{
    switch (rt) {
    case 2: launch_pair_rt<D, 2>(args, n_items, stream); break;
    case 4: launch_pair_rt<D, 4>(args, n_items, stream); break;
    case 6: launch_pair_rt<D, 6>(args, n_items, stream); break;
    default: return hipErrorInvalidValue;   // no such build; the planner never asks for it
    }
    return hipGetLastError();
}

hipError_t launch_attn_bf16_pair(int d, int rt, const AttnArgs &args, int n_items, hipStream_t stream)
{
    if (n_items <= 0)
        return hipSuccess;
    return d == 128 ? launch_pair_d<128>(rt, args, n_items, stream) : launch_pair_d<64>(rt, args, n_items, stream);
}

}  // namespace crkv
