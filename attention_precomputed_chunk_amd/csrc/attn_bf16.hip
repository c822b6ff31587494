// bf16 attention of query rows over a segment table of precomputed K/V
// chunks, with per-key impact partials, for gfx950 (CDNA4).
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
// Matrix-core layout (v_mfma_f32_16x16x32_bf16, 64 lanes; li = lane % 16,
// lg = lane / 16). Scores are taken as S^T = K . Q^T: A = 16 keys x 32 d from
// LDS, B = 32 d x 16 rows held in registers for the whole sweep. The
// accumulator gives lane (li, lg) row li and four keys. The A rows of the two
// 16-key subtiles of a 32-key tile are permuted so that lane (li, lg) ends up
// holding keys 8lg .. 8lg+7, which rounded to bf16 are exactly the B operand of
// O^T = V^T . P^T, so P never leaves registers. The V^T operand comes from V
// stored row-major in LDS through ds_read_b64_tr_b16: inside each 16-lane
// group, if lane j reads four bf16 B[j][0..3], lane i receives
// B[4e + i/4][i % 4] (e = 0..3), so lane j addresses V[key0 + j/4][d0 + 4(j%4)]
// and two such reads give lane i the eight keys of column d0 + i.
//
// On gfx950 the matrix cores and the vector ALU of a SIMD hardly overlap, so
// the kernel keeps both instruction streams short: no per-row-tile branches
// (each wave owns a compile-time number of 16-row tiles, padded rows are
// masked by an infinite lse), K/V tiles staged through 16 registers per
// thread, one barrier per 32-key tile.
//
// Work decomposition: one workgroup of 4 waves per (problem, KV head, block of
// 4 * RT row tiles). The rows of the G query heads sharing a KV head are
// packed as (query row j, head h) so one K/V tile in LDS serves the group.
#include <type_traits>

#include "device_util.h"

namespace crkv {

// K tile slot of 16-byte chunk `ch` of row `key`: the 16 keys one A operand
// reads (keys 8(i>>2) + 4s + (i&3)) land in 16 distinct slots.
template <int NCH>
__device__ __forceinline__ int kswz(int key)
{
    return NCH == 16 ? ((key & 3) | (((key >> 3) & 3) << 2)) : ((key & 3) | (((key >> 3) & 1) << 2));
}
// V tile: even XOR values keep each 32-byte pair of chunks together, and the
// rows one transposed read touches (4 consecutive keys, 8 for two lane
// groups) get distinct 32-byte bank groups.
template <int NCH>
__device__ __forceinline__ int vswz(int key)
{
    return NCH == 16 ? 2 * ((key & 3) | (((key >> 3) & 1) << 2)) : 2 * (key & 3);
}

// A key tile's descriptor held in scalar registers (passed by value so it is
// never demoted to scratch memory).
struct TileSR {
    gptr<const u32x4> K;
    gptr<const u32x4> V;
    int n_valid, key0, seg_len, seg_lo;
};

// A descriptor is eight dwords; lane l loads dword l % 8 with a vector load,
// one iteration before the dwords are moved to scalar registers, so the
// load's latency is covered by a tile of work. (A scalar load would count
// against lgkmcnt and be waited for with the next LDS read.)
__device__ __forceinline__ uint32_t load_tile(const KTile *tiles, int i, int lane)
{
    return as_global(reinterpret_cast<const uint32_t *>(tiles))[(size_t)i * 8 + (lane & 7)];
}

__device__ __forceinline__ TileSR to_sr(uint32_t raw)
{
    auto dw = [&](int j) { return (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)raw, j); };
    TileSR r;
    r.K = reinterpret_cast<gptr<const u32x4>>(dw(0) | (dw(1) << 32));
    r.V = reinterpret_cast<gptr<const u32x4>>(dw(2) | (dw(3) << 32));
    r.n_valid = (int)dw(4);
    r.key0 = (int)dw(5);
    r.seg_len = (int)dw(6);
    r.seg_lo = (int)dw(7);
    return r;
}

// One tile's K (and V) chunks in flight from global memory to LDS. Returned
// and passed by value so that it stays in registers.
template <int SLD>
struct Staged {
    u32x4 k[SLD];
    u32x4 v[SLD];
};

template <int NCH, int SLD, bool WITH_V>
__device__ __forceinline__ Staged<SLD> stage_load(TileSR kt, int kv_head, int tid)
{
    Staged<SLD> st;
    const size_t base = (size_t)kv_head * kt.seg_len * NCH;
#pragma unroll
    for (int i = 0; i < SLD; ++i) {
        const int cidx = tid + i * kThreads;
        const int key = min(cidx / NCH, kt.n_valid - 1);   // missing keys repeat a real one; masked later
        const int ch = cidx % NCH;
        st.k[i] = kt.K[base + (size_t)key * NCH + ch];
        if constexpr (WITH_V)
            st.v[i] = kt.V[base + (size_t)key * NCH + ch];
    }
    return st;
}

template <int NCH, int SLD, bool WITH_V>
__device__ __forceinline__ void stage_store(const Staged<SLD> st, unsigned char *lk, unsigned char *lv,
                                            int tid)
{
    constexpr int ROW = NCH * 16;
#pragma unroll
    for (int i = 0; i < SLD; ++i) {
        const int cidx = tid + i * kThreads;
        const int key = cidx / NCH, ch = cidx % NCH;
        *reinterpret_cast<u32x4 *>(lk + key * ROW + ((ch ^ kswz<NCH>(key)) << 4)) = st.k[i];
        if constexpr (WITH_V)
            *reinterpret_cast<u32x4 *>(lv + key * ROW + ((ch ^ vswz<NCH>(key)) << 4)) = st.v[i];
    }
}

template <int D, int RT, bool CROSS>
__global__ void __launch_bounds__(kThreads, 1) attn_bf16_kernel(const AttnArgs a)
{
    constexpr int KS = D / 32;                 // MFMA k-steps along d
    constexpr int DT = D / 16;                 // output d tiles
    constexpr int NCH = D / 8;                 // 16-byte chunks per row
    constexpr int ROW = 2 * D;                 // LDS bytes per K or V row
    constexpr int TILE = kKeyTile * ROW;       // LDS bytes per K (or V) tile
    constexpr int SLD = TILE / (kThreads * 16);  // staged chunks per thread (K or V)
    static_assert(kKeyTile == 32 && SLD >= 1, "tile geometry");

    __shared__ __attribute__((aligned(16))) unsigned char lds_k[2][TILE];
    __shared__ __attribute__((aligned(16))) unsigned char lds_v[2][TILE];
    __shared__ float lds_imp[2][kWaves][kKeyTile];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const ItemDesc it = a.items[blockIdx.x];
    if (it.n_rowtiles == 0)
        return;
    const ProbDesc pr = a.probs[it.prob];
    const int G = a.G;
    const float c = a.c_log2;
    const int packed_total = G * pr.rows;
    const int t0 = it.tile_begin + wave * RT;
    const int wave_min_pos = pr.pos0 + (t0 * kRowTile) / G;

    int row_pos[RT];
    bf16x8 qf[RT][KS];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
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
    const int kkey0 = 8 * (li >> 2) + (li & 3);          // A row li of subtile 0 (subtile 1: +4)
    const int ksw = kswz<NCH>(kkey0);                     // same for kkey0 + 4
    auto k_off = [&](int sub, int ks) { return (kkey0 + 4 * sub) * ROW + (((4 * ks + lg) ^ ksw) << 4); };
    auto v_off = [&](int dt, int r) {
        const int key = 8 * lg + 4 * r + (li >> 2);
        const int d = 16 * dt + 4 * (li & 3);
        return key * ROW + (((d >> 3) ^ vswz<NCH>(key)) << 4) + (d & 7) * 2;
    };

    const int n_kt = it.n_ktiles;
    // ---------------------------------------------------------------- sweep 1: row lse
    float row_m[RT], row_l[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        row_m[rt] = -INFINITY;
        row_l[rt] = 0.f;
    }
    auto sweep1_tile = [&](TileSR kt, int buf, auto mask_tag) {
        constexpr bool MASK = decltype(mask_tag)::value;
        bf16x8 kf[2][KS];
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                kf[sub][ks] = *reinterpret_cast<const bf16x8 *>(&lds_k[buf][k_off(sub, ks)]);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f}, s1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[0][ks], qf[rt][ks], s0, 0, 0, 0);
                s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[1][ks], qf[rt][ks], s1, 0, 0, 0);
            }
            if constexpr (MASK) {
                const int lim = min(kt.n_valid - 1, row_pos[rt] - kt.key0);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (8 * lg + e > lim)
                        s0[e] = -INFINITY;
                    if (8 * lg + 4 + e > lim)
                        s1[e] = -INFINITY;
                }
            }
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

    // Descriptors are loaded two tiles ahead of use and data one tile ahead;
    // a descriptor reaches scalar registers one iteration after its load.
    auto desc = [&](int tt) { return load_tile(pr.tiles, min(tt, n_kt - 1), lane); };
    if (n_kt > 0) {
        TileSR cur = to_sr(desc(0));
        uint32_t nraw = desc(1);
        stage_store<NCH, SLD, false>(stage_load<NCH, SLD, false>(cur, it.kv_head, tid), lds_k[0], lds_v[0], tid);
        __syncthreads();
        for (int tt = 0; tt < n_kt; ++tt) {
            const int buf = tt & 1;
            const bool more = tt + 1 < n_kt;
            const TileSR nxt = to_sr(nraw);
            nraw = desc(tt + 2);
            Staged<SLD> st;
            if (more)
                st = stage_load<NCH, SLD, false>(nxt, it.kv_head, tid);
            const bool need_mask = (cur.n_valid < kKeyTile) || (cur.key0 + cur.n_valid - 1 > wave_min_pos);
            if (need_mask)
                sweep1_tile(cur, buf, std::true_type{});
            else
                sweep1_tile(cur, buf, std::false_type{});
            if (more)
                stage_store<NCH, SLD, false>(st, lds_k[buf ^ 1], lds_v[buf ^ 1], tid);
            __syncthreads();
            cur = nxt;
        }
    }

    // Combine the four lane groups of each row into its log2-domain lse;
    // padded rows get +inf so every weight they would produce is 0.
    float lse2[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        float m = row_m[rt], l = row_l[rt];
        merge_state(m, l, __shfl_xor(m, 16), __shfl_xor(l, 16), c);
        merge_state(m, l, __shfl_xor(m, 32), __shfl_xor(l, 32), c);
        lse2[rt] = (row_pos[rt] < 0x3fffffff) ? m * c + __log2f(l) : INFINITY;
    }

    // ---------------------------------------------------------------- sweep 2: P.V and impact
    f32x4 o[RT][DT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
            o[rt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};

    const gptr<float> partial = as_global(pr.partial) + (size_t)it.slot * pr.n_keys;
    auto flush_impact = [&](int tt, TileSR kt, int buf) {
        if (wave == (tt & 3)) {
            if (lane < kt.n_valid)
                partial[kt.key0 + lane] = lds_imp[buf][0][lane] + lds_imp[buf][1][lane] +
                                          lds_imp[buf][2][lane] + lds_imp[buf][3][lane];
        }
    };
    auto sweep2_tile = [&](TileSR kt, int buf, auto mask_tag) {
        constexpr bool MASK = decltype(mask_tag)::value;
        bf16x8 kf[2][KS], vf[DT];
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                kf[sub][ks] = *reinterpret_cast<const bf16x8 *>(&lds_k[buf][k_off(sub, ks)]);
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
        for (int i = 0; i < 8; ++i)
            imp[i] = 0.f;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f}, s1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[0][ks], qf[rt][ks], s0, 0, 0, 0);
                s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[1][ks], qf[rt][ks], s1, 0, 0, 0);
            }
            if constexpr (MASK) {
                const int lim = min(kt.n_valid - 1, row_pos[rt] - kt.key0);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (8 * lg + e > lim)
                        s0[e] = -INFINITY;
                    if (8 * lg + 4 + e > lim)
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
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                o[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[dt], pb, o[rt][dt], 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
            imp[i] = row16_sum(imp[i]);
        if (li == 0) {
            float *dst = &lds_imp[buf][wave][8 * lg];
            *reinterpret_cast<float4 *>(dst) = make_float4(imp[0], imp[1], imp[2], imp[3]);
            *reinterpret_cast<float4 *>(dst + 4) = make_float4(imp[4], imp[5], imp[6], imp[7]);
        }
    };

    if (n_kt > 0) {
        TileSR cur = to_sr(desc(0)), prev = cur;
        uint32_t nraw = desc(1);
        stage_store<NCH, SLD, true>(stage_load<NCH, SLD, true>(cur, it.kv_head, tid), lds_k[0], lds_v[0], tid);
        __syncthreads();
        for (int tt = 0; tt < n_kt; ++tt) {
            const int buf = tt & 1;
            const bool more = tt + 1 < n_kt;
            const TileSR nxt = to_sr(nraw);
            nraw = desc(tt + 2);
            Staged<SLD> st;
            if (more)
                st = stage_load<NCH, SLD, true>(nxt, it.kv_head, tid);
            if (tt > 0)
                flush_impact(tt - 1, prev, buf ^ 1);
            const bool need_mask = (cur.n_valid < kKeyTile) || (cur.key0 + cur.n_valid - 1 > wave_min_pos);
            if (need_mask)
                sweep2_tile(cur, buf, std::true_type{});
            else
                sweep2_tile(cur, buf, std::false_type{});
            if (more)
                stage_store<NCH, SLD, true>(st, lds_k[buf ^ 1], lds_v[buf ^ 1], tid);
            __syncthreads();
            prev = cur;
            cur = nxt;
        }
        flush_impact(n_kt - 1, prev, (n_kt - 1) & 1);
    }

    // ---------------------------------------------------------------- epilogue: out rows
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
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

template <int D, int RT>
static void launch_rt(const AttnArgs &args, int n_items, hipStream_t stream)
{
    if constexpr (RT <= kMaxRowTilesCross) {
        if (args.cross) {
            hipLaunchKernelGGL((attn_bf16_kernel<D, RT, true>), dim3(n_items), dim3(kThreads), 0, stream, args);
            return;
        }
    }
    hipLaunchKernelGGL((attn_bf16_kernel<D, RT, false>), dim3(n_items), dim3(kThreads), 0, stream, args);
}

hipError_t launch_attn_bf16(int d, int rt, const AttnArgs &args, int n_items, hipStream_t stream)
{
    if (n_items <= 0)
        return hipSuccess;
    if (args.cross && rt > kMaxRowTilesCross)
        return hipErrorInvalidValue;   // no such build; the planner never asks for it
    if (d == 128) {
        if (rt == 7)
            launch_rt<128, 7>(args, n_items, stream);
        else if (rt == 5)
            launch_rt<128, 5>(args, n_items, stream);
        else
            launch_rt<128, 4>(args, n_items, stream);
    } else {
        if (rt == 7)
            launch_rt<64, 7>(args, n_items, stream);
        else if (rt == 5)
            launch_rt<64, 5>(args, n_items, stream);
        else
            launch_rt<64, 4>(args, n_items, stream);
    }
    return hipGetLastError();
}

}  // namespace crkv
