// The 8-bit K/V segment format and a decode step that reads it, for gfx950
// (CDNA4).
//
// Why: a decode step reads every cached K and V row once and does 4 d FLOPs
// per (head, key), so its time is the HBM time of the cache (the CacheGen
// summary: loading the cache dominates, and caches can be stored in a much
// smaller form; the page gives no codec). Values become signed 8-bit codes
// with float32 scales, about half the bytes of bf16:
//   scale = max over the group of |x| / 127,   code = round_half_even(x / scale)
// (float32 divisions, so the integer decision is the one an IEEE float32
// evaluation makes; an all-zero group gets scale 0 and zero codes). K has a
// group per (KV head, channel) over the segment's tokens, since cached keys
// carry a few large-magnitude channels; V a group per (KV head, token).
//
// quantize_q8_token_kernel (V): one row per d/8 lanes (8 values per lane),
// the row's maximum by lane shuffles, codes written as 8-byte pieces; a
// thread issues the loads of all its rows before the first is used.
// quantize_q8_channel_kernel (K): one workgroup per (segment, KV head); the
// channel maxima over the tokens are reduced through LDS, then the tokens are
// read a second time (from L2) and coded; four rows' loads in flight per
// thread in both passes.
//
// decode_q8_split_kernel: the split step of the bf16 decode
// (decode_bf16.hip) with 8-bit operands. The codes are small integers, exact
// in bf16, so they go to the matrix cores as they are and the scales are
// applied outside the products:
//   s_hi = (q_h * scale_K) . codeK_i / sqrt(d)   (q times the segment's channel
//          scales, formed once per segment as a bf16 pair hi + lo, so the
//          products carry about 16 significant bits: two MFMAs per k-step)
//   O_h  = sum_i (p_hi * scale_V(i)) codeV_i,     the sum of p_hi as usual.
// K codes go from global memory straight into A-operand registers: lane
// (li, lg) reads bytes [lg d/4, (lg + 1) d/4) of its key's row, and k-step ks
// of the MFMA takes d = lg d/4 + 8 ks + e, so Q's B operand is loaded with the
// same permutation of d (a contraction over d does not depend on its order).
// V codes are widened to bf16 into the wave's LDS tile in the layout the
// transposed reads of the bf16 kernel expect. The partials are the bf16
// decode's, merged by its merge kernel.
#include "attn_bf16_common.h"

namespace crkv {

// ---------------------------------------------------------------- quantize
template <int D>
__global__ void __launch_bounds__(kQ8Threads) quantize_q8_token_kernel(const Q8Args a)
{
    constexpr int LPR = D / 8;                   // lanes per row
    constexpr int RPP = kQ8Threads / LPR;        // rows per pass of the workgroup
    static_assert(64 % LPR == 0, "a row's lanes stay inside one wave");
    const Q8Item it = a.items[blockIdx.x];
    const Q8Seg sg = a.segs[it.seg];
    const int g = threadIdx.x % LPR;             // values 8g .. 8g+7 of the row
    const gptr<const u32x4> x = as_global(static_cast<const u32x4 *>(sg.x));
    const gptr<u32x2> codes = as_global(static_cast<u32x2 *>(sg.q8));
    const gptr<float> scales = as_global(reinterpret_cast<float *>(static_cast<unsigned char *>(sg.q8) +
                                                                   (size_t)sg.rows * D));
    constexpr int PER = kQ8RowsPerItem / RPP;   // rows per thread
    const int row_end = min(sg.rows, it.row0 + kQ8RowsPerItem);
    const int r0 = it.row0 + (int)threadIdx.x / LPR;
    u32x4 vs[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k)
        vs[k] = r0 + k * RPP < row_end ? x[(size_t)(r0 + k * RPP) * LPR + g] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int r = r0 + k * RPP;
        if (r >= row_end)   // the same for every lane of the row
            break;
        const u32x4 v = vs[k];
        float f[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            f[2 * q] = __uint_as_float(v[q] << 16);
            f[2 * q + 1] = __uint_as_float(v[q] & 0xFFFF0000u);
        }
        float amax = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            amax = fmaxf(amax, fabsf(f[e]));
#pragma unroll
        for (int o = 1; o < LPR; o <<= 1)
            amax = fmaxf(amax, __shfl_xor(amax, o));
        const float scale = amax / 127.0f;      // IEEE division
        uint32_t w[2] = {0u, 0u};
        if (scale > 0.f) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float q = fminf(fmaxf(__builtin_rintf(f[e] / scale), -127.f), 127.f);
                w[e / 4] |= ((uint32_t)(int)q & 0xFFu) << (8 * (e % 4));
            }
        }
        codes[(size_t)r * LPR + g] = u32x2{w[0], w[1]};
        if (g == 0)
            scales[r] = scale;
    }
}

template <int D>
__global__ void __launch_bounds__(kQ8Threads) quantize_q8_channel_kernel(const Q8Args a)
{
    constexpr int LPR = D / 8;                   // lanes per row
    constexpr int RG = kQ8Threads / LPR;         // row groups
    __shared__ float red[RG][D];
    __shared__ float sc[D];
    const Q8Item it = a.items[blockIdx.x];
    const Q8Seg sg = a.segs[it.seg];
    const int head = it.row0, len = sg.len;
    const int g = threadIdx.x % LPR, rg = threadIdx.x / LPR;   // channels 8g .. 8g+7
    const gptr<const u32x4> x = as_global(static_cast<const u32x4 *>(sg.x)) + (size_t)head * len * LPR;
    const gptr<u32x2> codes = as_global(static_cast<u32x2 *>(sg.q8)) + (size_t)head * len * LPR;
    const gptr<float> scales = as_global(reinterpret_cast<float *>(static_cast<unsigned char *>(sg.q8) +
                                                                   (size_t)sg.rows * D)) + (size_t)head * D;
    auto widen = [](const u32x4 v, float (&f)[8]) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            f[2 * q] = __uint_as_float(v[q] << 16);
            f[2 * q + 1] = __uint_as_float(v[q] & 0xFFFF0000u);
        }
    };
    float mx[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        mx[e] = 0.f;
    constexpr int UN = 4;                        // rows in flight per thread
    for (int r0 = rg; r0 < len; r0 += UN * RG) {
        u32x4 v[UN];
#pragma unroll
        for (int k = 0; k < UN; ++k)   // a missing row reads as zeros: no effect on a maximum
            v[k] = r0 + k * RG < len ? x[(size_t)(r0 + k * RG) * LPR + g] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int k = 0; k < UN; ++k) {
            float f[8];
            widen(v[k], f);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                mx[e] = fmaxf(mx[e], fabsf(f[e]));
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e)
        red[rg][8 * g + e] = mx[e];
    __syncthreads();
    if (threadIdx.x < D) {
        float m = red[0][threadIdx.x];
#pragma unroll
        for (int i = 1; i < RG; ++i)
            m = fmaxf(m, red[i][threadIdx.x]);
        const float s = m / 127.0f;              // IEEE division
        sc[threadIdx.x] = s;
        scales[threadIdx.x] = s;
    }
    __syncthreads();
    float s[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        s[e] = sc[8 * g + e];
    for (int r0 = rg; r0 < len; r0 += UN * RG) {
        u32x4 v[UN];
#pragma unroll
        for (int k = 0; k < UN; ++k)
            v[k] = r0 + k * RG < len ? x[(size_t)(r0 + k * RG) * LPR + g] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int k = 0; k < UN; ++k) {
            if (r0 + k * RG >= len)
                break;
            float f[8];
            widen(v[k], f);
            uint32_t w[2] = {0u, 0u};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float q = s[e] > 0.f ? fminf(fmaxf(__builtin_rintf(f[e] / s[e]), -127.f), 127.f) : 0.f;
                w[e / 4] |= ((uint32_t)(int)q & 0xFFu) << (8 * (e % 4));
            }
            codes[(size_t)(r0 + k * RG) * LPR + g] = u32x2{w[0], w[1]};
        }
    }
}

// Per-token (V) items, then per-channel (K) items, in one call.
hipError_t launch_quantize_q8(int d, const Q8Args &v_args, int n_v, const Q8Args &k_args, int n_k,
                              hipStream_t stream)
{
    if (n_v > 0) {
        if (d == 128)
            hipLaunchKernelGGL(quantize_q8_token_kernel<128>, dim3(n_v), dim3(kQ8Threads), 0, stream, v_args);
        else
            hipLaunchKernelGGL(quantize_q8_token_kernel<64>, dim3(n_v), dim3(kQ8Threads), 0, stream, v_args);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    if (n_k > 0) {
        if (d == 128)
            hipLaunchKernelGGL(quantize_q8_channel_kernel<128>, dim3(n_k), dim3(kQ8Threads), 0, stream, k_args);
        else
            hipLaunchKernelGGL(quantize_q8_channel_kernel<64>, dim3(n_k), dim3(kQ8Threads), 0, stream, k_args);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------- decode split over 8-bit segments
constexpr int kQ8DecodeThreads = kDecodeWaves * 64;

// Eight codes (two dwords, lowest byte first) widened to bf16, exactly.
__device__ __forceinline__ bf16x8 codes_bf16(uint32_t lo, uint32_t hi)
{
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        r[e] = (__bf16)(float)(int)(int8_t)(lo >> (8 * e));
        r[4 + e] = (__bf16)(float)(int)(int8_t)(hi >> (8 * e));
    }
    return r;
}

template <int D>
struct Q8Frags {
    u32x4 k[2][D / 64];                   // K codes of keys kkey0, kkey0 + 4: bytes [lg D/4, +D/4)
    u32x4 v[(kKeyTile * D / 16) / 64];    // this lane's 16-byte pieces of the V codes
    float vs[8];                          // V scales of keys 8 lg .. 8 lg + 7
};

template <int D>
__global__ void __launch_bounds__(kQ8DecodeThreads, 2) decode_q8_split_kernel(const DecodeArgs a)
{
    constexpr int KS = D / 32;
    constexpr int DT = D / 16;
    constexpr int NCH = D / 8;                 // 16-byte bf16 chunks per LDS row
    constexpr int ROW = 2 * D;                 // LDS bytes per (widened) V row
    constexpr int TILE = kKeyTile * ROW;
    constexpr int PPR = D / 16;                // 16-byte code pieces per row
    constexpr int VP = (kKeyTile * PPR) / 64;  // V pieces per lane per tile
    constexpr int KP = D / 64;                 // K code pieces per lane per key
    constexpr int MERGE_BYTES = kDecodeWaves * D * kRowTile * 4;
    constexpr int SMEM = kDecodeWaves * TILE > MERGE_BYTES ? kDecodeWaves * TILE : MERGE_BYTES;
    __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];
    __shared__ float lds_m[kDecodeWaves][kRowTile], lds_l[kDecodeWaves][kRowTile];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 15, lg = lane >> 4;
    const DecodeItem it = a.items[blockIdx.x];
    const ProbDesc pr = a.probs[it.prob];
    const int G = a.G;
    const float c = a.c_log2;
    unsigned char *vt = smem + wave * TILE;

    // Q^T of the G heads (columns >= G are zero), with d permuted as the K
    // codes are read: k-step ks, lane group lg holds d = lg D/4 + 8 ks + e.
    // qh + ql is Q times the current segment's K channel scales.
    bf16x8 qh[KS], ql[KS];
    int qs_seg = -1;                   // seg_lo of the segment qh, ql were made for
    const bool q_valid = li < G;
    const gptr<const u32x4> qrow = as_global(reinterpret_cast<const u32x4 *>(pr.Q)) +
                                   (size_t)(q_valid ? it.kv_head * G + li : 0) * NCH;

    const int kkey0 = 8 * (li >> 2) + (li & 3);   // A row li of subtile 0 (subtile 1: +4)
    auto v_off = [&](int dt, int r) {
        const int key = 8 * lg + 4 * r + (li >> 2);
        const int dd = 16 * dt + 4 * (li & 3);
        return key * ROW + (((dd >> 3) ^ vswz<NCH>(key)) << 4) + (dd & 7) * 2;
    };
    // Tile t: codes and scales from global memory. The tile's K (V) pointer is
    // its segment's buffer at code row t0 = key0 - seg_lo of KV head 0; the
    // segment's scales start H_kv * seg_len * D bytes into the buffer.
    auto fetch = [&](TileSR kt) {
        Q8Frags<D> f;
        const int t0 = kt.key0 - kt.seg_lo;
        const size_t head_rows = (size_t)it.kv_head * kt.seg_len;
        const gptr<const unsigned char> kc =
            reinterpret_cast<gptr<const unsigned char>>(kt.K) + head_rows * D;
        const gptr<const unsigned char> vc =
            reinterpret_cast<gptr<const unsigned char>>(kt.V) + head_rows * D;
        const size_t to_scales = (size_t)a.H_kv * kt.seg_len * D - (size_t)t0 * D;
        const gptr<const float> vsc =
            reinterpret_cast<gptr<const float>>(reinterpret_cast<gptr<const unsigned char>>(kt.V) + to_scales) +
            head_rows + t0;
        const int last = kt.n_valid - 1;   // missing keys repeat a real one; masked later
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            const int key = min(kkey0 + 4 * sub, last);
#pragma unroll
            for (int j = 0; j < KP; ++j)
                f.k[sub][j] = *reinterpret_cast<gptr<const u32x4>>(kc + (size_t)key * D + lg * (D / 4) + 16 * j);
        }
#pragma unroll
        for (int i = 0; i < VP; ++i) {
            const int pc = lane + 64 * i;
            const int key = min(pc / PPR, last);
            f.v[i] = *reinterpret_cast<gptr<const u32x4>>(vc + (size_t)key * D + 16 * (pc % PPR));
        }
#pragma unroll
        for (int e = 0; e < 8; ++e)
            f.vs[e] = vsc[min(8 * lg + e, last)];
        return f;
    };
    // qh, ql for the segment of tile kt: its K scales are [H_kv][D] floats
    // after the codes; this lane needs channels lg D/4 .. lg D/4 + D/4 - 1.
    auto scale_q = [&](TileSR kt) {
        const int t0 = kt.key0 - kt.seg_lo;
        const gptr<const f32x4> ksc = reinterpret_cast<gptr<const f32x4>>(
            reinterpret_cast<gptr<const unsigned char>>(kt.K) + (size_t)a.H_kv * kt.seg_len * D - (size_t)t0 * D +
            ((size_t)it.kv_head * D + lg * (D / 4)) * sizeof(float));
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 q = __builtin_bit_cast(bf16x8, q_valid ? qrow[KS * lg + ks] : u32x4{0u, 0u, 0u, 0u});
            const f32x4 s0 = ksc[2 * ks], s1 = ksc[2 * ks + 1];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = (float)q[e] * (e < 4 ? s0[e] : s1[e - 4]);
                qh[ks][e] = (__bf16)x;
                ql[ks][e] = (__bf16)(x - (float)qh[ks][e]);
            }
        }
        qs_seg = kt.seg_lo;
    };
    auto put_v = [&](const Q8Frags<D> &f) {
#pragma unroll
        for (int i = 0; i < VP; ++i) {
            const int pc = lane + 64 * i;
            const int key = pc / PPR, cc = 2 * (pc % PPR);
            const bf16x8 lo = codes_bf16(f.v[i][0], f.v[i][1]);
            const bf16x8 hi = codes_bf16(f.v[i][2], f.v[i][3]);
            *reinterpret_cast<bf16x8 *>(vt + key * ROW + ((cc ^ vswz<NCH>(key)) << 4)) = lo;
            *reinterpret_cast<bf16x8 *>(vt + key * ROW + (((cc + 1) ^ vswz<NCH>(key)) << 4)) = hi;
        }
    };

    f32x4 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
        o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, l = 0.f;   // row li's running max (scaled score) and this lane's partial sum

    auto desc = [&](int t) { return to_sr(load_tile(pr.tiles, it.tile_begin + min(t, it.n_tiles - 1), lane)); };
    if (wave < it.n_tiles) {
        TileSR cur = desc(wave);
        Q8Frags<D> fc = fetch(cur);
        put_v(fc);
        for (int t = wave; t < it.n_tiles; t += kDecodeWaves) {
            bf16x8 vf[DT];
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(vt + v_off(dt, 0)));
                const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(vt + v_off(dt, 1)));
                vf[dt] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
            const bool more = t + kDecodeWaves < it.n_tiles;
            const TileSR nxt = desc(t + kDecodeWaves);
            Q8Frags<D> fn;
            if (more)
                fn = fetch(nxt);

            bf16x8 kf[2][KS];
#pragma unroll
            for (int sub = 0; sub < 2; ++sub)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    kf[sub][ks] = codes_bf16(fc.k[sub][ks / 2][2 * (ks % 2)], fc.k[sub][ks / 2][2 * (ks % 2) + 1]);
            if (cur.seg_lo != qs_seg)   // wave-uniform: a new segment's scales
                scale_q(cur);
            Spair sc = scores<KS>(kf, qh);
            const Spair sl = scores<KS>(kf, ql);
            sc.s0 += sl.s0;
            sc.s1 += sl.s1;
            if (cur.n_valid < kKeyTile)
                mask_scores_decode(sc, cur.n_valid - 1, lg);
            float tmax = fmaxf(fmaxf(fmaxf(sc.s0[0], sc.s0[1]), fmaxf(sc.s0[2], sc.s0[3])),
                               fmaxf(fmaxf(sc.s1[0], sc.s1[1]), fmaxf(sc.s1[2], sc.s1[3])));
            tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
            const float mn = fmaxf(m, tmax);               // finite: every tile has a real key
            const float alpha = exp2_hw((m - mn) * c);     // 0 on the first tile (m = -inf)
            const float mc = mn * c;
            float p[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                p[e] = exp2_hw(__builtin_fmaf(sc.s0[e], c, -mc));
                p[4 + e] = exp2_hw(__builtin_fmaf(sc.s1[e], c, -mc));
            }
            const float sum = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
            l = __builtin_fmaf(l, alpha, sum);
            m = mn;
            bf16x8 pb;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                pb[i] = (__bf16)(p[i] * fc.vs[i]);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                o[dt] *= alpha;
                o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[dt], pb, o[dt], 0, 0, 0);
            }
            if (more) {
                put_v(fn);   // after this tile's V reads, in the wave's LDS order
                fc = fn;
            }
            cur = nxt;
        }
    }
    // The four lanes of a row hold partial sums over their keys.
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);

    // ---------------------------------------------------------------- merge the four waves
    __syncthreads();   // every wave is done with its V tile: smem becomes the merge area
    float *mo = reinterpret_cast<float *>(smem);   // [wave][d][row]
    if (lg == 0) {
        lds_m[wave][li] = m;
        lds_l[wave][li] = l;
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            mo[(wave * D + 16 * dt + 4 * lg + e) * kRowTile + li] = o[dt][e];
    __syncthreads();
    float *part = a.part + (size_t)it.part * (size_t)G * (2 + D);
    for (int idx = tid; idx < G * D; idx += kQ8DecodeThreads) {
        const int r = idx / D, dd = idx % D;
        float M = lds_m[0][r];
#pragma unroll
        for (int w = 1; w < kDecodeWaves; ++w)
            M = fmaxf(M, lds_m[w][r]);
        float L = 0.f, O = 0.f;
#pragma unroll
        for (int w = 0; w < kDecodeWaves; ++w) {
            const float f = exp2_hw((lds_m[w][r] - M) * c);   // 0 for a wave without tiles
            L = __builtin_fmaf(lds_l[w][r], f, L);
            O = __builtin_fmaf(mo[(w * D + dd) * kRowTile + r], f, O);
        }
        part[2 * G + r * D + dd] = O;
        if (dd == 0) {
            part[2 * r] = M;
            part[2 * r + 1] = L;
        }
    }
}

hipError_t launch_decode_merge(int d, const DecodeArgs &args, int n_pairs, hipStream_t stream);

hipError_t launch_decode_q8(int d, const DecodeArgs &args, int n_items, int n_pairs, hipStream_t stream)
{
    if (n_items <= 0)
        return hipSuccess;
    if (d == 128)
        hipLaunchKernelGGL(decode_q8_split_kernel<128>, dim3(n_items), dim3(kQ8DecodeThreads), 0, stream, args);
    else
        hipLaunchKernelGGL(decode_q8_split_kernel<64>, dim3(n_items), dim3(kQ8DecodeThreads), 0, stream, args);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    return launch_decode_merge(d, args, n_pairs, stream);
}

}  // namespace crkv
