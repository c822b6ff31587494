// fp32 attention over a segment table of precomputed K/V chunks (same
// definition as the bf16 kernels: TurboRAG summary, causal attention over
// K_combined = Concat(K^(1..m), K^(Q)); CacheBlend summary, Impact equation),
// and the deterministic combine of the impact partials.
#include "device_util.h"

namespace crkv {

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
    float4 qf[Q4];
    {
        const float4 *qrow = reinterpret_cast<const float4 *>(pr.Q) + (size_t)(valid ? row_off : 0) * (D / 4);
#pragma unroll
        for (int q = 0; q < Q4; ++q)
            qf[q] = valid ? qrow[lg * Q4 + q] : make_float4(0.f, 0.f, 0.f, 0.f);
    }

    // S^T for 16 keys of a tile (keys 16*sb + li as A rows).
    auto scores = [&](const KTile &kt, int sb) -> f32x4 {
        const int key = 16 * sb + li;
        const bool kv = key < kt.n_valid;
        const float4 *krow = reinterpret_cast<const float4 *>(kt.K) +
                             ((size_t)it.kv_head * kt.seg_len + (kv ? key : 0)) * (D / 4);
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
        for (int sb = 0; sb < kKeyTile / 16; ++sb) {
            if (16 * sb >= kt.n_valid)
                break;
            const f32x4 s = scores(kt, sb);
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
        const bool own_segment = row_pos >= kt.seg_lo && row_pos < kt.seg_lo + kt.seg_len;
        const float wt = (a.cross && own_segment) ? 0.f : 1.f;
        for (int sb = 0; sb < kKeyTile / 16; ++sb) {
            if (16 * sb >= kt.n_valid)
                break;
            const f32x4 s = scores(kt, sb);
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
                const float *vrow = reinterpret_cast<const float *>(kt.V) +
                                    ((size_t)it.kv_head * kt.seg_len + (kv ? key : 0)) * D;
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

// impact[i] = sum over slots of partial[slot][i] for the slots whose key
// range reaches i. One workgroup per (64 keys, problem): wave w sums slots
// [w*S/4, (w+1)*S/4) in order, then the four wave sums are added in wave
// order, so the result is deterministic (no atomics anywhere). Entries past a
// slot's key range (causal row blocks end early) are never written and are
// selected away after the load.
constexpr int kCombineKeys = 64;

__global__ void __launch_bounds__(256) impact_combine_kernel(const ProbDesc *probs)
{
    __shared__ float red[4][kCombineKeys];
    const ProbDesc pr = probs[blockIdx.y];
    const int k0 = blockIdx.x * kCombineKeys;
    if (k0 >= pr.n_keys)
        return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int i = k0 + lane;
    const int s_lo = (int)((int64_t)wave * pr.n_slots / 4), s_hi = (int)((int64_t)(wave + 1) * pr.n_slots / 4);
    // Loads are unconditional (every slot row is allocated in full) and the
    // extent test only selects, so consecutive slots' loads overlap.
    const int ii = min(i, pr.n_keys - 1);
    float acc = 0.f;
#pragma unroll 8
    for (int s = s_lo; s < s_hi; ++s) {
        // select on the bits: an unwritten entry may hold any pattern
        const int v = __float_as_int(pr.partial[(size_t)s * pr.n_keys + ii]);
        acc += __int_as_float((i < pr.slot_end[s]) ? v : 0);
    }
    red[wave][lane] = acc;
    __syncthreads();
    if (wave == 0 && i < pr.n_keys)
        pr.impact[i] = ((red[0][lane] + red[1][lane]) + red[2][lane]) + red[3][lane];
}

// ------------------------------------------------------------------ launchers

hipError_t launch_attn_f32(int d, const AttnArgs &args, int n_items, hipStream_t stream)
{
    if (n_items <= 0)
        return hipSuccess;
    if (d == 128)
        hipLaunchKernelGGL((attn_f32_kernel<128>), dim3(n_items), dim3(64), 0, stream, args);
    else
        hipLaunchKernelGGL((attn_f32_kernel<64>), dim3(n_items), dim3(64), 0, stream, args);
    return hipGetLastError();
}

hipError_t launch_combine(const ProbDesc *probs, int n_probs, int max_keys, hipStream_t stream)
{
    if (n_probs <= 0 || max_keys <= 0)
        return hipSuccess;
    const dim3 grid((max_keys + kCombineKeys - 1) / kCombineKeys, n_probs);
    hipLaunchKernelGGL(impact_combine_kernel, grid, dim3(256), 0, stream, probs);
    return hipGetLastError();
}

}  // namespace crkv
