// Attention of query rows over a segment table of precomputed K/V chunks,
// with per-key impact, for gfx950 (CDNA4).
//
// What is computed (TurboRAG summary: K_combined = Concat(K^(1..m), K^(Q)) and
// the causal attention equation; CacheBlend summary: the Impact equation and
// the selective-recompute listing's softmax and column sum):
//   s_ji  = q_j . k_i / sqrt(d)            for keys at position <= the row's
//   p_ji  = exp(s_ji - lse_j),  lse_j = log sum_i exp(s_ji)
//   out_j = sum_i p_ji v_i
//   imp_i = sum over heads and counted rows of p_ji
//
// Exact impact needs every row's final lse before any column sum, so each
// workgroup sweeps its keys twice: sweep 1 computes the row lse, sweep 2
// recomputes the scores, forms p in fp32, accumulates the impact column sums
// from the fp32 p, and runs P.V on the matrix cores with p rounded to bf16.
//
// MFMA layout (v_mfma_f32_16x16x32_bf16, 64 lanes; li = lane % 16,
// lg = lane / 16). The product is taken as S^T = K . Q^T: A = 16 keys x 32 d,
// B = 32 d x 16 rows, and the accumulator gives lane (li, lg) the row li and
// four keys. Within each 32-key block the A rows of the two 16-key subtiles
// are permuted so that lane (li, lg) ends up holding keys 8lg .. 8lg+7 of the
// block. Those eight fp32 weights, rounded to bf16, are exactly the B operand
// of O^T = V^T . P^T, so P never leaves registers. V^T is produced by
// transposing V on its way into LDS.
//
// Work decomposition: one workgroup of 4 waves per (problem, KV head, block of
// up to 4 * 5 row tiles). The rows of the G query heads that share a KV head
// are packed as (query row j, head h) so that one K/V tile in LDS serves the
// whole group. Each wave owns up to 5 row tiles and keeps their Q fragments
// and output accumulators in registers for the whole sweep.
#include <hip/hip_runtime.h>

#include "crkv_internal.h"

namespace crkv {

typedef __bf16 bf16x8 __attribute__((__vector_size__(16)));
typedef float f32x4 __attribute__((__vector_size__(16)));

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

__device__ __forceinline__ uint32_t u4get(const uint4 &v, int i)
{
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Combine two (max, sum) softmax states given in the log2 domain scale c.
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

// K tile: row `key` holds d contiguous; 16-byte chunk ch sits at slot
// ch ^ kswz(key) so that the 16 keys one MFMA A operand reads land in
// distinct banks.
template <int NCH>
__device__ __forceinline__ int kswz(int key)
{
    return (key & 3) | (((key >> 3) & ((NCH >> 2) - 1)) << 2);
}
// V^T tile: row d holds 64 keys; 16-byte chunk c (8 keys) sits at c ^ vswz(d).
__device__ __forceinline__ int vswz(int d) { return (d ^ (d >> 3)) & 7; }

template <int D, int RT>
__global__ void __launch_bounds__(kThreads, 1) attn_bf16_kernel(const AttnArgs a)
{
    constexpr int KS = D / 32;             // MFMA k-steps along d
    constexpr int DT = D / 16;             // output d tiles
    constexpr int NCH = D / 8;             // 16-byte chunks per K/V row
    constexpr int KROW = D * 2;            // LDS bytes per K row
    constexpr int KBYTES = kKeyTile * KROW;
    constexpr int VROW = kKeyTile * 2;     // LDS bytes per V^T row
    constexpr int VBYTES = D * VROW;
    constexpr int KLD = kKeyTile * NCH / kThreads;  // K chunks per thread per tile
    constexpr int KPT = kKeyTile * NCH / kThreads;  // keys per thread in V staging
    static_assert(KLD >= 1 && (KPT == 2 || KPT == 4), "tile geometry");

    __shared__ __attribute__((aligned(16))) unsigned char lds_k[2][KBYTES];
    __shared__ __attribute__((aligned(16))) unsigned char lds_v[2][VBYTES];
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

    // This wave's row tiles.
    const int per = it.n_rowtiles / kWaves, extra = it.n_rowtiles % kWaves;
    const int my_nt = per + (wave < extra ? 1 : 0);
    const int my_t0 = it.tile_begin + wave * per + (wave < extra ? wave : extra);
    const int wave_min_pos = pr.pos0 + (my_t0 * kRowTile) / G;

    int row_off[RT], row_pos[RT], row_seg[RT];
    uint4 qf[RT][KS];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int r = (my_t0 + rt) * kRowTile + li;
        const bool valid = (rt < my_nt) && (r < packed_total);
        const int j = r / G;
        const int h = it.kv_head * G + (r - j * G);
        row_off[rt] = valid ? h * pr.rows + j : -1;
        row_pos[rt] = valid ? pr.pos0 + j : 0x3fffffff;
        row_seg[rt] = a.cross && valid ? segment_of(pr.segs, pr.n_seg, pr.pos0 + j) : -1;
        const uint4 *qrow = reinterpret_cast<const uint4 *>(pr.Q) + (size_t)(valid ? row_off[rt] : 0) * NCH;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qf[rt][ks] = valid ? qrow[4 * ks + lg] : make_uint4(0, 0, 0, 0);
    }

    // Per-lane LDS offsets of the MFMA operand fragments.
    int koff[2];                      // K rows of subtile 0/1 inside a 32-key block
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
        const int key = 8 * (li >> 2) + 4 * sub + (li & 3);
        koff[sub] = key * KROW;
    }
    const int ksw = kswz<NCH>(8 * (li >> 2) + (li & 3));

    const int n_kt = it.n_ktiles;
    uint4 kreg[KLD], vreg[KPT];

    auto load_tile = [&](int tt, bool with_v) {
        const KTile kt = pr.tiles[tt];
        const SegDesc sg = pr.segs[kt.seg];
        const size_t base = ((size_t)it.kv_head * sg.len + kt.local0) * NCH;
        const uint4 *Kb = reinterpret_cast<const uint4 *>(sg.K) + base;
#pragma unroll
        for (int i = 0; i < KLD; ++i) {
            const int cidx = tid + i * kThreads;
            const int key = cidx / NCH, ch = cidx % NCH;
            kreg[i] = key < kt.n_valid ? Kb[key * NCH + ch] : make_uint4(0, 0, 0, 0);
        }
        if (with_v) {
            const uint4 *Vb = reinterpret_cast<const uint4 *>(sg.V) + base;
            const int ch = tid % NCH, kg = tid / NCH;
#pragma unroll
            for (int e = 0; e < KPT; ++e) {
                const int key = kg * KPT + e;
                vreg[e] = key < kt.n_valid ? Vb[key * NCH + ch] : make_uint4(0, 0, 0, 0);
            }
        }
    };
    auto store_tile = [&](int buf, bool with_v) {
#pragma unroll
        for (int i = 0; i < KLD; ++i) {
            const int cidx = tid + i * kThreads;
            const int key = cidx / NCH, ch = cidx % NCH;
            *reinterpret_cast<uint4 *>(&lds_k[buf][key * KROW + ((ch ^ kswz<NCH>(key)) << 4)]) = kreg[i];
        }
        if (with_v) {
            const int ch = tid % NCH, kg = tid / NCH;
            const int k0 = kg * KPT;
#pragma unroll
            for (int dl = 0; dl < 8; ++dl) {
                const int dd = ch * 8 + dl;
                uint32_t hv[KPT];
#pragma unroll
                for (int e = 0; e < KPT; ++e) {
                    const uint32_t w = u4get(vreg[e], dl >> 1);
                    hv[e] = (dl & 1) ? (w >> 16) : (w & 0xFFFFu);
                }
                const int off = dd * VROW + (((k0 >> 3) ^ vswz(dd)) << 4) + (k0 & 7) * 2;
                if constexpr (KPT == 4) {
                    *reinterpret_cast<uint2 *>(&lds_v[buf][off]) =
                        make_uint2(hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16));
                } else {
                    *reinterpret_cast<uint32_t *>(&lds_v[buf][off]) = hv[0] | (hv[1] << 16);
                }
            }
        }
    };

    float row_m[RT], row_l[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        row_m[rt] = -INFINITY;
        row_l[rt] = 0.f;
    }

    // ---------------------------------------------------------------- sweep 1: row lse
    if (n_kt > 0) {
        load_tile(0, false);
        store_tile(0, false);
    }
    __syncthreads();
    for (int tt = 0; tt < n_kt; ++tt) {
        const int buf = tt & 1;
        if (tt + 1 < n_kt)
            load_tile(tt + 1, false);
        const KTile kt = pr.tiles[tt];
        const bool need_mask = (kt.n_valid < kKeyTile) || (kt.key0 + kt.n_valid - 1 > wave_min_pos);
        bf16x8 kf[2][2][KS];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int sub = 0; sub < 2; ++sub)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    kf[kb][sub][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(
                        &lds_k[buf][kb * 32 * KROW + koff[sub] + (((4 * ks + lg) ^ ksw) << 4)]));
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            if (rt >= my_nt)
                break;
            f32x4 s[2][2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int sub = 0; sub < 2; ++sub) {
                    s[kb][sub] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks)
                        s[kb][sub] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            kf[kb][sub][ks], __builtin_bit_cast(bf16x8, qf[rt][ks]), s[kb][sub], 0, 0, 0);
                }
            if (need_mask) {
                const int lim = min(kt.n_valid - 1, row_pos[rt] - kt.key0);
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (32 * kb + 8 * lg + 4 * sub + e > lim)
                                s[kb][sub][e] = -INFINITY;
            }
            float tmax = row_m[rt];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int sub = 0; sub < 2; ++sub)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        tmax = fmaxf(tmax, s[kb][sub][e]);
            const float mu = (tmax == -INFINITY) ? 0.f : tmax;
            const float mc = mu * c;
            float sum = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int sub = 0; sub < 2; ++sub)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        sum += exp2_hw(__builtin_fmaf(s[kb][sub][e], c, -mc));
            row_l[rt] = row_l[rt] * exp2_hw(__builtin_fmaf(row_m[rt], c, -mc)) + sum;
            row_m[rt] = tmax;
        }
        if (tt + 1 < n_kt)
            store_tile(buf ^ 1, false);
        __syncthreads();
    }

    // Combine the four lane groups of each row into the row's log2-domain lse.
    float lse2[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        float m = row_m[rt], l = row_l[rt];
        merge_state(m, l, __shfl_xor(m, 16), __shfl_xor(l, 16), c);
        merge_state(m, l, __shfl_xor(m, 32), __shfl_xor(l, 32), c);
        lse2[rt] = (row_off[rt] >= 0) ? m * c + __log2f(l) : INFINITY;
    }

    // ---------------------------------------------------------------- sweep 2: P.V and impact
    f32x4 o[RT][DT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
            o[rt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};

    float *partial = pr.partial + (size_t)it.slot * pr.n_keys;
    auto flush_impact = [&](int tt, int buf) {
        // one wave writes the tile's impact partial, summed over the 4 waves
        if (wave == (tt & 3)) {
            const KTile kt = pr.tiles[tt];
            if (lane < kt.n_valid) {
                const float v = lds_imp[buf][0][lane] + lds_imp[buf][1][lane] +
                                lds_imp[buf][2][lane] + lds_imp[buf][3][lane];
                partial[kt.key0 + lane] = v;
            }
        }
    };

    if (n_kt > 0) {
        load_tile(0, true);
        store_tile(0, true);
    }
    __syncthreads();
    for (int tt = 0; tt < n_kt; ++tt) {
        const int buf = tt & 1;
        if (tt + 1 < n_kt)
            load_tile(tt + 1, true);
        if (tt > 0)
            flush_impact(tt - 1, buf ^ 1);
        const KTile kt = pr.tiles[tt];
        const bool need_mask = (kt.n_valid < kKeyTile) || (kt.key0 + kt.n_valid - 1 > wave_min_pos);
        // impact weight of each row for this tile's segment
        float wt[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
            wt[rt] = (a.cross && row_seg[rt] == kt.seg) ? 0.f : 1.f;

#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            bf16x8 kf[2][KS], vf[DT];
#pragma unroll
            for (int sub = 0; sub < 2; ++sub)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    kf[sub][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(
                        &lds_k[buf][kb * 32 * KROW + koff[sub] + (((4 * ks + lg) ^ ksw) << 4)]));
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const int dd = 16 * dt + li;
                vf[dt] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(
                    &lds_v[buf][dd * VROW + (((4 * kb + lg) ^ vswz(dd)) << 4)]));
            }
            float imp[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                imp[i] = 0.f;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                if (rt >= my_nt)
                    break;
                f32x4 s[2];
#pragma unroll
                for (int sub = 0; sub < 2; ++sub) {
                    s[sub] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks)
                        s[sub] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            kf[sub][ks], __builtin_bit_cast(bf16x8, qf[rt][ks]), s[sub], 0, 0, 0);
                }
                if (need_mask) {
                    const int lim = min(kt.n_valid - 1, row_pos[rt] - kt.key0);
#pragma unroll
                    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (32 * kb + 8 * lg + 4 * sub + e > lim)
                                s[sub][e] = -INFINITY;
                }
                float p[8];
#pragma unroll
                for (int sub = 0; sub < 2; ++sub)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        p[4 * sub + e] = exp2_hw(__builtin_fmaf(s[sub][e], c, -lse2[rt]));
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    imp[i] = __builtin_fmaf(p[i], wt[rt], imp[i]);
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
                float *dst = &lds_imp[buf][wave][32 * kb + 8 * lg];
                *reinterpret_cast<float4 *>(dst) = make_float4(imp[0], imp[1], imp[2], imp[3]);
                *reinterpret_cast<float4 *>(dst + 4) = make_float4(imp[4], imp[5], imp[6], imp[7]);
            }
        }
        if (tt + 1 < n_kt)
            store_tile(buf ^ 1, true);
        __syncthreads();
    }
    if (n_kt > 0)
        flush_impact(n_kt - 1, (n_kt - 1) & 1);

    // ---------------------------------------------------------------- epilogue: out rows
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        if (row_off[rt] < 0)
            continue;
        uint16_t *orow = reinterpret_cast<uint16_t *>(pr.out) + (size_t)row_off[rt] * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            __bf16 b0 = (__bf16)o[rt][dt][0], b1 = (__bf16)o[rt][dt][1];
            __bf16 b2 = (__bf16)o[rt][dt][2], b3 = (__bf16)o[rt][dt][3];
            const uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, b0) |
                                ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
            const uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, b2) |
                                ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
            *reinterpret_cast<uint2 *>(orow + 16 * dt + 4 * lg) = make_uint2(lo, hi);
        }
    }
}

// fp32 inputs: one wave per (problem, KV head, 16-row tile), operands read
// straight from global memory (L2), v_mfma_f32_16x16x4_f32 for both products
// so no reduced-precision path is involved. Same two sweeps as above. In a
// 4-wide k-step, lane group lg supplies contraction index lg; for Q.K^T the
// d axis is split so that lane group lg walks d = (D/4)*lg + ks.
template <int D>
__global__ void __launch_bounds__(64) attn_f32_kernel(const AttnArgs a)
{
    constexpr int Q4 = D / 16;    // float4 per lane of a Q or K row quarter
    constexpr int DT = D / 16;
    const int lane = threadIdx.x & 63;
    const int li = lane & 15, lg = lane >> 4;
    const ItemDesc it = a.items[blockIdx.x];
    if (it.n_rowtiles == 0)
        return;
    const ProbDesc pr = a.probs[it.prob];
    const int G = a.G;
    const float c = a.c_log2;
    const int packed_total = G * pr.rows;

    const int r = it.tile_begin * kRowTile + li;
    const bool valid = r < packed_total;
    const int j = r / G;
    const int h = it.kv_head * G + (r - j * G);
    const int row_off = valid ? h * pr.rows + j : -1;
    const int row_pos = valid ? pr.pos0 + j : 0x3fffffff;
    const int row_seg = a.cross && valid ? segment_of(pr.segs, pr.n_seg, row_pos) : -1;
    float4 qf[Q4];
    {
        const float4 *qrow = reinterpret_cast<const float4 *>(pr.Q) + (size_t)(valid ? row_off : 0) * (D / 4);
#pragma unroll
        for (int q = 0; q < Q4; ++q)
            qf[q] = valid ? qrow[lg * Q4 + q] : make_float4(0.f, 0.f, 0.f, 0.f);
    }

    // S^T for 16 keys of a tile (keys 16*sb + li as A rows).
    auto scores = [&](const KTile &kt, const SegDesc &sg, int sb) -> f32x4 {
        const int key = 16 * sb + li;
        const bool kv = key < kt.n_valid;
        const float4 *krow = reinterpret_cast<const float4 *>(sg.K) +
                             ((size_t)it.kv_head * sg.len + kt.local0 + (kv ? key : 0)) * (D / 4);
        f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < Q4; ++q) {
            const float4 kk = kv ? krow[lg * Q4 + q] : make_float4(0.f, 0.f, 0.f, 0.f);
            s = __builtin_amdgcn_mfma_f32_16x16x4f32(kk.x, qf[q].x, s, 0, 0, 0);
            s = __builtin_amdgcn_mfma_f32_16x16x4f32(kk.y, qf[q].y, s, 0, 0, 0);
            s = __builtin_amdgcn_mfma_f32_16x16x4f32(kk.z, qf[q].z, s, 0, 0, 0);
            s = __builtin_amdgcn_mfma_f32_16x16x4f32(kk.w, qf[q].w, s, 0, 0, 0);
        }
        const int lim = min(kt.n_valid - 1, row_pos - kt.key0);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (16 * sb + 4 * lg + e > lim)
                s[e] = -INFINITY;
        return s;
    };

    const int n_kt = it.n_ktiles;
    float m = -INFINITY, l = 0.f;
    for (int tt = 0; tt < n_kt; ++tt) {
        const KTile kt = pr.tiles[tt];
        const SegDesc sg = pr.segs[kt.seg];
        for (int sb = 0; sb < kKeyTile / 16; ++sb) {
            if (16 * sb >= kt.n_valid)
                break;
            const f32x4 s = scores(kt, sg, sb);
            const float tmax = fmaxf(fmaxf(fmaxf(m, s[0]), fmaxf(s[1], s[2])), s[3]);
            const float mu = (tmax == -INFINITY) ? 0.f : tmax;
            const float mc = mu * c;
            float sum = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                sum += exp2_hw(__builtin_fmaf(s[e], c, -mc));
            l = l * exp2_hw(__builtin_fmaf(m, c, -mc)) + sum;
            m = tmax;
        }
    }
    merge_state(m, l, __shfl_xor(m, 16), __shfl_xor(l, 16), c);
    merge_state(m, l, __shfl_xor(m, 32), __shfl_xor(l, 32), c);
    const float lse2 = valid ? m * c + __log2f(l) : INFINITY;

    f32x4 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
        o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float *partial = pr.partial + (size_t)it.slot * pr.n_keys;
    for (int tt = 0; tt < n_kt; ++tt) {
        const KTile kt = pr.tiles[tt];
        const SegDesc sg = pr.segs[kt.seg];
        const float wt = (a.cross && row_seg == kt.seg) ? 0.f : 1.f;
        for (int sb = 0; sb < kKeyTile / 16; ++sb) {
            if (16 * sb >= kt.n_valid)
                break;
            const f32x4 s = scores(kt, sg, sb);
            float p[4], imp[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                p[e] = exp2_hw(__builtin_fmaf(s[e], c, -lse2));
                imp[e] = row16_sum(p[e] * wt);
            }
            // O^T += V^T P^T: k-step e pairs key 16*sb + 4*lg + e with p[e]
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int key = 16 * sb + 4 * lg + e;
                const bool kv = key < kt.n_valid;
                const float *vrow = reinterpret_cast<const float *>(sg.V) +
                                    ((size_t)it.kv_head * sg.len + kt.local0 + (kv ? key : 0)) * D;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const float vv = kv ? vrow[16 * dt + li] : 0.f;
                    o[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(vv, p[e], o[dt], 0, 0, 0);
                }
            }
            if (li == 0) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int key = 16 * sb + 4 * lg + e;
                    if (key < kt.n_valid)
                        partial[kt.key0 + key] = imp[e];
                }
            }
        }
    }
    if (row_off >= 0) {
        float *orow = reinterpret_cast<float *>(pr.out) + (size_t)row_off * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
            *reinterpret_cast<float4 *>(orow + 16 * dt + 4 * lg) =
                make_float4(o[dt][0], o[dt][1], o[dt][2], o[dt][3]);
    }
}

// impact[i] = sum over slots (fixed order) of partial[slot][i] for the slots
// whose key range reaches i. Deterministic: no atomics anywhere.
__global__ void __launch_bounds__(256) impact_combine_kernel(const ProbDesc *probs)
{
    const ProbDesc pr = probs[blockIdx.y];
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= pr.n_keys)
        return;
    float acc = 0.f;
    for (int s = 0; s < pr.n_slots; ++s)
        if (i < pr.slot_end[s])
            acc += pr.partial[(size_t)s * pr.n_keys + i];
    pr.impact[i] = acc;
}

// ------------------------------------------------------------------ launchers

hipError_t launch_attn(bool bf16, int d, const AttnArgs &args, int n_items, hipStream_t stream)
{
    if (n_items <= 0)
        return hipSuccess;
    const dim3 grid(n_items);
    if (bf16) {
        if (d == 128)
            hipLaunchKernelGGL((attn_bf16_kernel<128, kRowTilesBf16>), grid, dim3(kThreads), 0, stream, args);
        else
            hipLaunchKernelGGL((attn_bf16_kernel<64, kRowTilesBf16>), grid, dim3(kThreads), 0, stream, args);
    } else {
        if (d == 128)
            hipLaunchKernelGGL((attn_f32_kernel<128>), grid, dim3(64), 0, stream, args);
        else
            hipLaunchKernelGGL((attn_f32_kernel<64>), grid, dim3(64), 0, stream, args);
    }
    return hipGetLastError();
}

hipError_t launch_combine(const ProbDesc *probs, int n_probs, int max_keys, hipStream_t stream)
{
    if (n_probs <= 0 || max_keys <= 0)
        return hipSuccess;
    const dim3 grid((max_keys + 255) / 256, n_probs);
    hipLaunchKernelGGL(impact_combine_kernel, grid, dim3(256), 0, stream, probs);
    return hipGetLastError();
}

}  // namespace crkv
