// One decode step over the segment table, bf16, for gfx950 (CDNA4).
//
// The query row of each head is the newest token, at the last position of the
// concatenation, so it sees every key (TurboRAG summary: the generation loop
// appends each generated token's K/V to the cache). out_h = sum_i p_hi v_i,
// p_hi = exp(s_hi - lse_h), s_hi = q_h . k_i / sqrt(d). No impact.
//
// A decode step reads every K and V row once and does 4 d FLOPs per (head,
// key): it is bound by HBM, not by the matrix cores. The keys of each
// (problem, KV head) are split into ranges of 32-key tiles; the split kernel
// runs one workgroup per range, the merge kernel one per (problem, KV head).
//
// Split kernel: 4 waves, wave w takes tiles w, w + 4, ... of the range, each
// with its own online softmax, so the waves never wait for one another inside
// the loop. The G query heads of the KV head form the 16 columns of one MFMA
// row tile (columns >= G are zero Q and are never stored), and the operand
// layouts are those of attn_bf16_common.h: K goes from global memory straight
// into A-operand registers (16-byte chunks, 64 contiguous bytes per key and
// lane quad), V goes through the wave's own LDS tile for the transposed
// ds_read_b64_tr_b16 reads. The next tile's loads are in flight while the
// current one is computed. At the end the four waves' states are merged in
// LDS and written as one partial: per head (max, sum) and the output row
// scaled to that max.
//
// Merge kernel: for each (problem, KV head), the heads' overall max and sum
// come from the partials' (max, sum); each partial's weight per head is
// staged in LDS, and every output element sums its partials in range order
// (deterministic) and is written in bf16.
#include "attn_bf16_common.h"

namespace crkv {

constexpr int kDecodeThreads = kDecodeWaves * 64;

template <int D>
struct DecodeFrags {
    bf16x8 k[2][D / 32];              // K fragments (A operands of S^T = K Q^T)
    u32x4 v[(kKeyTile * D / 8) / 64];   // this lane's 16-byte chunks of the V tile
};

template <int D>
__global__ void __launch_bounds__(kDecodeThreads, 2) decode_split_kernel(const DecodeArgs a)
{
    constexpr int KS = D / 32;
    constexpr int DT = D / 16;
    constexpr int NCH = D / 8;                 // 16-byte chunks per row
    constexpr int ROW = 2 * D;                 // LDS bytes per V row
    constexpr int TILE = kKeyTile * ROW;
    constexpr int VCH = (kKeyTile * NCH) / 64; // V chunks per lane per tile
    constexpr int MERGE_BYTES = kDecodeWaves * D * kRowTile * 4;
    constexpr int SMEM = kDecodeWaves * TILE > MERGE_BYTES ? kDecodeWaves * TILE : MERGE_BYTES;
    // Per-wave V tiles during the loop; the merge area afterwards.
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

    // Q^T of the G heads (columns >= G are zero): the heads of KV head
    // it.kv_head are packed rows 0 .. G-1 of row tile 0 (one row per head).
    bf16x8 qf[KS];
    int row_pos;
    {
        ItemDesc q_it{};
        q_it.kv_head = it.kv_head;
        load_q_rows<KS>(pr, q_it, G, 0, li, lg, qf, row_pos);
    }

    const int kkey0 = 8 * (li >> 2) + (li & 3);   // A row li of subtile 0 (subtile 1: +4)
    auto v_off = [&](int dt, int r) {
        const int key = 8 * lg + 4 * r + (li >> 2);
        const int dd = 16 * dt + 4 * (li & 3);
        return key * ROW + (((dd >> 3) ^ vswz<NCH>(key)) << 4) + (dd & 7) * 2;
    };
    // Tile t of the range: K fragments and V chunks from global memory.
    auto fetch = [&](TileSR kt) {
        DecodeFrags<D> f;
        const size_t head = (size_t)it.kv_head * kt.seg_len * NCH;
        const int last = kt.n_valid - 1;   // missing keys repeat a real one; masked later
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            const int key = min(kkey0 + 4 * sub, last);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                f.k[sub][ks] = __builtin_bit_cast(bf16x8, (u32x4)kt.K[head + (size_t)key * NCH + 4 * ks + lg]);
        }
#pragma unroll
        for (int i = 0; i < VCH; ++i) {
            const int ch = lane + 64 * i;
            const int key = min(ch / NCH, last);
            f.v[i] = kt.V[head + (size_t)key * NCH + ch % NCH];
        }
        return f;
    };
    auto put_v = [&](const DecodeFrags<D> &f) {
#pragma unroll
        for (int i = 0; i < VCH; ++i) {
            const int ch = lane + 64 * i;
            const int key = ch / NCH, cc = ch % NCH;
            *reinterpret_cast<u32x4 *>(vt + key * ROW + ((cc ^ vswz<NCH>(key)) << 4)) = f.v[i];
        }
    };

    f32x4 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
        o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, l = 0.f;   // row li's running max (raw score) and this lane's partial sum

    auto desc = [&](int t) { return to_sr(load_tile(pr.tiles, it.tile_begin + min(t, it.n_tiles - 1), lane)); };
    if (wave < it.n_tiles) {
        TileSR cur = desc(wave);
        DecodeFrags<D> fc = fetch(cur);
        put_v(fc);
        for (int t = wave; t < it.n_tiles; t += kDecodeWaves) {
            // V^T fragments of the current tile (written at the end of the
            // previous iteration; a wave's LDS accesses complete in order)
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
            DecodeFrags<D> fn;
            if (more)
                fn = fetch(nxt);

            Spair sc = scores<KS>(fc.k, qf);
            if (cur.n_valid < kKeyTile)
                mask_scores_decode(sc, cur.n_valid - 1, lg);
            float tmax = fmaxf(fmaxf(fmaxf(sc.s0[0], sc.s0[1]), fmaxf(sc.s0[2], sc.s0[3])),
                               fmaxf(fmaxf(sc.s1[0], sc.s1[1]), fmaxf(sc.s1[2], sc.s1[3])));
            tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
            const float mn = fmaxf(m, tmax);               // finite: every tile has a real key
            const float alpha = exp2_hw((m - mn) * c);     // 0 on the first tile (m = -inf)
            const float mc = mn * c;
            float p[8], sum = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                p[e] = exp2_hw(__builtin_fmaf(sc.s0[e], c, -mc));
                p[4 + e] = exp2_hw(__builtin_fmaf(sc.s1[e], c, -mc));
            }
#pragma unroll
            for (int i = 0; i < 8; ++i)
                sum += p[i];
            l = __builtin_fmaf(l, alpha, sum);
            m = mn;
            bf16x8 pb;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                pb[i] = (__bf16)p[i];
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
    for (int idx = tid; idx < G * D; idx += kDecodeThreads) {
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

// Partials a merge workgroup stages in LDS at once (more are merged in chunks).
constexpr int kMergeChunk = 64;

template <int D>
__global__ void __launch_bounds__(256) decode_merge_kernel(const DecodeArgs a)
{
    __shared__ float w_lds[kMergeChunk][kDecodeMaxGroup];   // weight of partial p for head r
    __shared__ float s_max[kDecodeMaxGroup], s_sum[kDecodeMaxGroup];
    const DecodePair pp = a.pairs[blockIdx.x];
    const ProbDesc pr = a.probs[pp.prob];
    const int G = a.G;
    const float c = a.c_log2;
    const size_t stride = (size_t)G * (2 + D);
    const float *base = a.part + (size_t)pp.part_begin * stride;
    const int tid = threadIdx.x;
    // the overall max and sum of each head, from the partials' (max, sum)
    if (tid < G) {
        float M = -INFINITY;
        for (int p = 0; p < pp.n_parts; ++p)
            M = fmaxf(M, base[p * stride + 2 * tid]);
        float L = 0.f;
        for (int p = 0; p < pp.n_parts; ++p)
            L = __builtin_fmaf(base[p * stride + 2 * tid + 1], exp2_hw((base[p * stride + 2 * tid] - M) * c), L);
        s_max[tid] = M;
        s_sum[tid] = L;
    }
    __syncthreads();
    float acc[(kDecodeMaxGroup * D + 255) / 256];
#pragma unroll
    for (int i = 0; i < (kDecodeMaxGroup * D + 255) / 256; ++i)
        acc[i] = 0.f;
    for (int p0 = 0; p0 < pp.n_parts; p0 += kMergeChunk) {
        const int np = min(kMergeChunk, pp.n_parts - p0);
        for (int x = tid; x < np * G; x += 256) {
            const int p = x / G, r = x % G;
            w_lds[p][r] = exp2_hw((base[(p0 + p) * stride + 2 * r] - s_max[r]) * c) / s_sum[r];
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < (kDecodeMaxGroup * D + 255) / 256; ++i) {
            const int idx = tid + 256 * i;
            if (idx < G * D) {
                const int r = idx / D;
                float o = acc[i];
                for (int p = 0; p < np; ++p)
                    o = __builtin_fmaf(base[(p0 + p) * stride + 2 * G + idx], w_lds[p][r], o);
                acc[i] = o;
            }
        }
        __syncthreads();
    }
    const gptr<__bf16> out = as_global(reinterpret_cast<__bf16 *>(pr.out));
#pragma unroll
    for (int i = 0; i < (kDecodeMaxGroup * D + 255) / 256; ++i) {
        const int idx = tid + 256 * i;
        if (idx < G * D) {
            const int r = idx / D, dd = idx % D;
            out[(size_t)(pp.kv_head * G + r) * D + dd] = (__bf16)acc[i];
        }
    }
}

// The merge alone (also used after the split step over 8-bit segments).
hipError_t launch_decode_merge(int d, const DecodeArgs &args, int n_pairs, hipStream_t stream)
{
    if (n_pairs <= 0)
        return hipSuccess;
    if (d == 128)
        hipLaunchKernelGGL(decode_merge_kernel<128>, dim3(n_pairs), dim3(256), 0, stream, args);
    else
        hipLaunchKernelGGL(decode_merge_kernel<64>, dim3(n_pairs), dim3(256), 0, stream, args);
    return hipGetLastError();
}

hipError_t launch_decode_bf16(int d, const DecodeArgs &args, int n_items, int n_pairs, hipStream_t stream)
{
    if (n_items <= 0)
        return hipSuccess;
    if (d == 128) {
        hipLaunchKernelGGL(decode_split_kernel<128>, dim3(n_items), dim3(kDecodeThreads), 0, stream, args);
        hipLaunchKernelGGL(decode_merge_kernel<128>, dim3(n_pairs), dim3(256), 0, stream, args);
    } else {
        hipLaunchKernelGGL(decode_split_kernel<64>, dim3(n_items), dim3(kDecodeThreads), 0, stream, args);
        hipLaunchKernelGGL(decode_merge_kernel<64>, dim3(n_pairs), dim3(256), 0, stream, args);
    }
    return hipGetLastError();
}

}  // namespace crkv
