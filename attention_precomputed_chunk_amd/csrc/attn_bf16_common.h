// Helpers shared by the gfx950 bf16 attention kernels: LDS tile layout, key
// tile descriptors, global-to-LDS staging and the score MFMAs.
//
// Matrix-core layout (v_mfma_f32_16x16x32_bf16, 64 lanes; li = lane % 16,
// lg = lane / 16). Scores are taken as S^T = K . Q^T: A = 16 keys x 32 d from
// LDS (subtile s of a 32-key tile: keys 16 s .. 16 s + 15, in order), B =
// 32 d x 16 rows held in registers for the whole sweep. The accumulator gives
// lane (li, lg) row li and keys 16 s + 4 lg + e (e < 4) of subtile s; a
// lane's eight scores of a tile (s = 0, 1), rounded to bf16, are exactly its
// B operand of O^T = V^T . P^T when k index 8 lg + 4 s + e stands for key
// 16 s + 4 lg + e. The V^T operand comes from V stored row-major in LDS
// through ds_read_b64_tr_b16: inside each 16-lane group, if lane j reads four
// bf16 B[j][0..3], lane i receives B[4e + i/4][i % 4] (e = 0..3), so lane j
// of group lg addresses V[16 r + 4 lg + j/4][d0 + 4(j%4)] in read r = 0, 1,
// and the two reads give lane i the keys of its k indices for column d0 + i.
//
// LDS tiles: K and V rows are 2D bytes padded to 2D + 32, an odd number of
// 32-byte units (9 at d = 128, 5 at d = 64). The padding, not a swizzle,
// spreads the rows over the banks, so each fragment read of a lane is one
// per-lane base plus a compile-time offset. A K read (16 bytes of row
// 16 s + li at column chunk 4 ks + lg: consecutive rows in the lanes of a
// group), a transposed V read (8 bytes of row 16 r + 4 lg + li/4) and the
// staging writes (whole rows) meet no bank conflict at this stride; in-bounds
// probes on gfx950 measured conflicts on K reads with rows padded by 16, 48
// or 64 bytes or unpadded, and on V reads padded by 16 or 64.
#pragma once
#include "device_util.h"

namespace crkv {

constexpr int kWsThreads = 2 * kWaves * 64;   // pair kernel: a producer and a consumer wave per SIMD

// XOR swizzle of the decode kernels' V tiles (16-byte chunk index of row
// `key`): even values keep each 32-byte pair of chunks together, and the
// rows one transposed read touches (4 consecutive keys, 8 for two lane
// groups) get distinct 32-byte bank groups.
template <int NCH>
__host__ __device__ constexpr int vswz(int key)
{
    return NCH == 16 ? 2 * ((key & 3) | (((key >> 3) & 1) << 2)) : 2 * (key & 3);
}

// LDS row strides and tile sizes of the attention kernels (NCH = D / 8
// 16-byte chunks of data per row).
template <int NCH>
constexpr int kRowK = NCH * 16 + 32;
template <int NCH>
constexpr int kRowV = NCH * 16 + 32;
template <int NCH>
constexpr int kTileK = kKeyTile * kRowK<NCH>;
template <int NCH>
constexpr int kTileV = kKeyTile * kRowV<NCH>;

// Lane (li, lg)'s LDS byte offsets inside a tile: its K fragment of subtile
// `sub` and k step `ks`, and its transposed V read `r` of d block dt.
template <int NCH>
__device__ __forceinline__ int k_frag_off(int li, int lg, int sub, int ks)
{
    return (16 * sub + li) * kRowK<NCH> + (4 * ks + lg) * 16;
}
template <int NCH>
__device__ __forceinline__ int v_frag_off(int li, int lg, int r, int dt)
{
    return (16 * r + 4 * lg + (li >> 2)) * kRowV<NCH> + (16 * dt + 4 * (li & 3)) * 2;
}
// Key (inside its tile) of accumulator element e of subtile s in lane group lg.
__device__ __forceinline__ int acc_key(int lg, int s, int e) { return 16 * s + 4 * lg + e; }
// The first of the two keys whose impact totals row16_sum8 leaves in lane
// (li, lg) of a group (elements 2(li/4), 2(li/4) + 1 of its eight).
__device__ __forceinline__ int imp_key(int li, int lg) { return 4 * lg + 2 * (li >> 2) + 12 * (li >> 3); }

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

// One key tile's K (and V) 16-byte chunks in flight from global memory to LDS,
// spread over NT threads: thread t moves chunks t + i NT (i < PER). Chunk index
// x < CH is K chunk x, else V chunk x - CH; chunk c of a tile is key c / NCH,
// column chunk c % NCH. Returned and passed by value so that it stays in
// registers.
template <int NCH, bool WITH_V, int NT>
struct Staged {
    static constexpr int CH = kKeyTile * NCH;
    static constexpr int TOTAL = WITH_V ? 2 * CH : CH;
    static constexpr int PER = (TOTAL + NT - 1) / NT;
    static_assert(!WITH_V || CH % NT == 0, "K and V chunks split evenly over the threads");
    u32x4 c[PER];
};

// A thread's fixed part of the staging, computed once. Thread t moves the
// chunks t + i NT: with NT a multiple of NCH its column chunk ch = t % NCH is
// the same for every i and its key advances by KS = NT / NCH rows per i, so
// the LDS byte offset of chunk i is the thread's first offset plus the
// compile-time i KS times the row stride. The global side clamps the key to
// the tile's last valid one (a min and a shift-or per chunk).
// WITH_V stages K then V of one tile; otherwise K alone.
template <int NCH, bool WITH_V, int NT>
struct Stager {
    using S = Staged<NCH, WITH_V, NT>;
    static constexpr int KS = NT / NCH;
    static_assert(NT % NCH == 0, "a thread keeps its column chunk");
    static constexpr bool is_v(int i) { return WITH_V && i * NT >= S::CH; }
    static constexpr int rel(int i) { return is_v(i) ? i - S::CH / NT : i; }   // chunk step inside K or V
    static constexpr bool all_valid = S::TOTAL % NT == 0;

    uint32_t kb, vb;    // LDS byte offsets of the thread's first K and V chunks
    bool last_ok;       // chunk PER - 1 exists (always, when all_valid)
    int k0, ch;

    __device__ __forceinline__ explicit Stager(int t)
    {
        k0 = t / NCH;
        ch = t % NCH;
        kb = (uint32_t)(k0 * kRowK<NCH> + ch * 16);
        vb = (uint32_t)(k0 * kRowV<NCH> + ch * 16);
        last_ok = all_valid || t + (S::PER - 1) * NT < S::TOTAL;
    }
    __device__ __forceinline__ bool has(int i) const { return i < S::PER - 1 || last_ok; }
    __device__ __forceinline__ uint32_t klds(int i) const { return kb + (uint32_t)(rel(i) * KS * kRowK<NCH>); }
    __device__ __forceinline__ uint32_t vlds(int i) const { return vb + (uint32_t)(rel(i) * KS * kRowV<NCH>); }

    // Row `key` of KV head g of the tile's segment starts g * seg_len rows past
    // the tile's base; keys past n_valid repeat the last real key (masked
    // later). Full and partial tiles share this one address form: with a
    // second form for full tiles in its own branch, the compiler's wait-count
    // pass took that branch's loads as possibly in flight where the other form
    // reuses their registers, and made every chunk load wait for all earlier
    // loads (the next tiles' descriptors and the previous tile's chunks).
    __device__ __forceinline__ S load(TileSR kt, int kv_head) const
    {
        S st;
        const size_t head = (size_t)kv_head * kt.seg_len * NCH;
        const gptr<const unsigned char> kbase = reinterpret_cast<gptr<const unsigned char>>(kt.K + head);
        const gptr<const unsigned char> vbase = reinterpret_cast<gptr<const unsigned char>>(kt.V + head);
        const int last = kt.n_valid - 1;
#pragma unroll
        for (int i = 0; i < S::PER; ++i)
            if (has(i)) {
                const int key = min(k0 + rel(i) * KS, last);
                st.c[i] = *reinterpret_cast<gptr<const u32x4>>((is_v(i) ? vbase : kbase) +
                                                               (uint32_t)((key * NCH + ch) * 16));
            }
        return st;
    }

    __device__ __forceinline__ void store(const S st, unsigned char *lk, unsigned char *lv) const
    {
#pragma unroll
        for (int i = 0; i < S::PER; ++i)
            if (has(i))
                *reinterpret_cast<u32x4 *>(is_v(i) ? lv + vlds(i) : lk + klds(i)) = st.c[i];
    }

    // A K-only stager moving the same chunks of the tile's V instead (into
    // a V tile, whose rows have the V stride).
    __device__ __forceinline__ S load_v(TileSR kt, int kv_head) const
    {
        static_assert(!WITH_V, "K-only stager");
        TileSR v = kt;
        v.K = kt.V;
        return load(v, kv_head);
    }
    __device__ __forceinline__ void store_v(const S st, unsigned char *lv) const
    {
        static_assert(!WITH_V, "K-only stager");
#pragma unroll
        for (int i = 0; i < S::PER; ++i)
            if (has(i))
                *reinterpret_cast<u32x4 *>(lv + vlds(i)) = st.c[i];
    }
};

// Eight codes (two dwords, lowest byte first) times float32 scales.
__device__ __forceinline__ void codes_times(uint32_t lo, uint32_t hi, const float *sc, float *x)
{
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        x[e] = (float)(int)(int8_t)(lo >> (8 * e)) * sc[e];
        x[4 + e] = (float)(int)(int8_t)(hi >> (8 * e)) * sc[4 + e];
    }
}

// Key tiles of segments in the 8-bit format (codes [H_kv][len][D] int8, then
// float32 scales: [H_kv][D] per channel for K, [H_kv][len] per token for V).
// Staging widens a tile into the bf16 tiles the matrix cores read:
//   K: x = code * scale[channel] in float32, stored as the pair hi = bf16(x)
//      (tile lk) and lo = bf16(x - hi) (tile lkl): Q . hi + Q . lo carries K
//      to about 17 significant bits, as the impact's tolerance needs;
//   V: bf16(code * scale[token]), one rounding (P . V is already rounded to
//      bf16 operands).
// Thread t < CH moves the 16 codes of chunk t (key t / (D/16), channels
// 16 (t % (D/16)) ..) of K and, with WITH_V, of V; the tile's scales come
// with it. A tile descriptor's K (V) pointer is its segment's buffer at code
// row key0 - seg_lo of KV head 0; the segment's scales start
// H_kv * seg_len * D bytes into that buffer.
template <int D, bool WITH_V, int NT>
struct StagedQ8 {
    u32x4 kc;
    f32x4 ks[4];
    u32x4 vc;
    float vs;
};

template <int D, bool WITH_V, int NT>
struct StagerQ8 {
    static constexpr int CPR = D / 16;          // 16-byte code chunks per row
    static constexpr int CH = kKeyTile * CPR;   // code chunks per tile
    static constexpr int NCH = D / 8;           // 16-byte bf16 chunks per row
    static_assert(CH <= NT, "one code chunk per thread");
    using S = StagedQ8<D, WITH_V, NT>;
    bool active;
    int key, c16;
    uint32_t lk0, lk1, lv0, lv1;   // LDS byte offsets of the chunk's two bf16 halves

    __device__ __forceinline__ explicit StagerQ8(int t)
    {
        active = t < CH;
        key = t / CPR;
        c16 = t % CPR;
        const int ch0 = 2 * c16, ch1 = 2 * c16 + 1;
        lk0 = (uint32_t)(key * kRowK<NCH> + ch0 * 16);
        lk1 = (uint32_t)(key * kRowK<NCH> + ch1 * 16);
        lv0 = (uint32_t)(key * kRowV<NCH> + ch0 * 16);
        lv1 = (uint32_t)(key * kRowV<NCH> + ch1 * 16);
    }

    // Keys past n_valid repeat the last real key (masked later).
    __device__ __forceinline__ S load(TileSR kt, int kv_head, int H_kv) const
    {
        S st;
        if (!active)
            return st;
        const int t0 = kt.key0 - kt.seg_lo;
        const int row = min(key, kt.n_valid - 1);
        const size_t head_rows = (size_t)kv_head * kt.seg_len;
        const size_t to_scales = (size_t)H_kv * kt.seg_len * D - (size_t)t0 * D;
        const gptr<const unsigned char> kb = reinterpret_cast<gptr<const unsigned char>>(kt.K);
        st.kc = *reinterpret_cast<gptr<const u32x4>>(kb + (head_rows + row) * D + 16 * c16);
        const gptr<const f32x4> ksc =
            reinterpret_cast<gptr<const f32x4>>(kb + to_scales + ((size_t)kv_head * D + 16 * c16) * sizeof(float));
#pragma unroll
        for (int j = 0; j < 4; ++j)
            st.ks[j] = ksc[j];
        if constexpr (WITH_V) {
            const gptr<const unsigned char> vb = reinterpret_cast<gptr<const unsigned char>>(kt.V);
            st.vc = *reinterpret_cast<gptr<const u32x4>>(vb + (head_rows + row) * D + 16 * c16);
            st.vs = reinterpret_cast<gptr<const float>>(vb + to_scales)[head_rows + t0 + row];
        }
        return st;
    }

    __device__ __forceinline__ void store(const S st, unsigned char *lk, unsigned char *lkl,
                                          unsigned char *lv) const
    {
        if (!active)
            return;
        float ksc[16];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                ksc[4 * j + e] = st.ks[j][e];
        float x[16];
        codes_times(st.kc[0], st.kc[1], ksc, x);
        codes_times(st.kc[2], st.kc[3], ksc + 8, x + 8);
        bf16x8 h0, h1, l0, l1;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            h0[e] = (__bf16)x[e];
            h1[e] = (__bf16)x[8 + e];
            l0[e] = (__bf16)(x[e] - (float)h0[e]);
            l1[e] = (__bf16)(x[8 + e] - (float)h1[e]);
        }
        *reinterpret_cast<bf16x8 *>(lk + lk0) = h0;
        *reinterpret_cast<bf16x8 *>(lk + lk1) = h1;
        *reinterpret_cast<bf16x8 *>(lkl + lk0) = l0;
        *reinterpret_cast<bf16x8 *>(lkl + lk1) = l1;
        if constexpr (WITH_V) {
            float vsc[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                vsc[e] = st.vs;
            float y[16];
            codes_times(st.vc[0], st.vc[1], vsc, y);
            codes_times(st.vc[2], st.vc[3], vsc, y + 8);
            bf16x8 v0, v1;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                v0[e] = (__bf16)y[e];
                v1[e] = (__bf16)y[8 + e];
            }
            *reinterpret_cast<bf16x8 *>(lv + lv0) = v0;
            *reinterpret_cast<bf16x8 *>(lv + lv1) = v1;
        }
    }
};

// S^T of one 16-row tile against the two 16-key subtiles of a key tile.
// Sweep 1 keeps per (row, lane group) a reference maximum m and
// l = sum of exp2((s - m) * c) over the keys seen so far, with m <= their
// maximum. An unmasked key tile is summed against the current m; the exact
// maximum is taken again (and l rescaled) only when some lane's sum over the
// tile exceeds 2^32, i.e. a score lies more than about 29 above m in log2
// units, which includes a row's first tile (m = -inf gives an infinite sum).
// lse = m * c + log2(l) is the same quantity either way; skipping the
// per-tile maximum and rescale removes a third of sweep 1's vector work
// (used by the one-wave kernel, whose sweep 1 is vector-bound; with two
// waves per SIMD the pair kernel measured no difference).
constexpr float kLseRescaleBound = 4294967296.0f;   // 2^32

struct Spair {
    f32x4 s0, s1;
};

template <int KS>
__device__ __forceinline__ Spair scores(const bf16x8 (&kf)[2][KS], const bf16x8 (&q)[KS])
{
    Spair r;
    r.s0 = f32x4{0.f, 0.f, 0.f, 0.f};
    r.s1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        r.s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[0][ks], q[ks], r.s0, 0, 0, 0);
        r.s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[1][ks], q[ks], r.s1, 0, 0, 0);
    }
    return r;
}

// Scores past the tile's valid keys or past the row's causal limit (`lim`,
// relative to the tile's first key) become -inf. mask_scores takes the
// attention kernels' key order (acc_key); mask_scores_decode the decode
// kernels', whose A rows of subtile s are keys 8(i/4) + 4s + i%4, so that
// element e of subtile s in lane group lg is key 8 lg + 4 s + e.
__device__ __forceinline__ void mask_scores(Spair &s, int lim, int lg)
{
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if (acc_key(lg, 0, e) > lim)
            s.s0[e] = -INFINITY;
        if (acc_key(lg, 1, e) > lim)
            s.s1[e] = -INFINITY;
    }
}
__device__ __forceinline__ void mask_scores_decode(Spair &s, int lim, int lg)
{
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if (8 * lg + e > lim)
            s.s0[e] = -INFINITY;
        if (8 * lg + 4 + e > lim)
            s.s1[e] = -INFINITY;
    }
}

// Log2-domain lse of packed row `local` of an item's row block, from the
// pass-1 states of the block's ranges merged in range order (the same value
// in every range's item of the block).
__device__ __forceinline__ float merged_lse(const AttnArgs &a, const ItemDesc &it, int local, float c)
{
    const gptr<const f32x2> st = as_global(reinterpret_cast<const f32x2 *>(a.state)) + (size_t)it.state + local;
    const f32x2 s0 = st[0];
    float m = s0.x, l = s0.y;
    for (int r = 1; r < it.n_ranges; ++r) {
        const f32x2 s = st[(size_t)r * a.cap_rows];
        merge_state(m, l, s.x, s.y, c);
    }
    return m * c + __log2f(l);
}

// Q^T fragments of row tile t: packed row r = 16 t + li is query row r / G of
// head kv_head * G + r % G; rows past the packed total are padding (zero Q,
// position beyond every key).
template <int KS>
__device__ __forceinline__ void load_q_rows(const ProbDesc &pr, const ItemDesc &it, int G, int t, int li,
                                            int lg, bf16x8 (&q)[KS], int &row_pos)
{
    constexpr int NCH = KS * 4;
    const int r = t * kRowTile + li;
    const bool valid = r < G * pr.rows;
    const int j = r / G;
    const int h = it.kv_head * G + (r - j * G);
    row_pos = valid ? pr.pos0 + j : 0x3fffffff;
    const gptr<const u32x4> qrow =
        as_global(reinterpret_cast<const u32x4 *>(pr.Q)) + (size_t)(valid ? h * pr.rows + j : 0) * NCH;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const u32x4 v = valid ? qrow[4 * ks + lg] : u32x4{0u, 0u, 0u, 0u};
        q[ks] = __builtin_bit_cast(bf16x8, v);
    }
}

}  // namespace crkv
