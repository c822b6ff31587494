// Drives the host side of libcrkv (validation, planning, budget, format
// sizes) without a GPU, for the AddressSanitizer / UndefinedBehaviorSanitizer
// build of crkv_api.hip made by tests/test_sanitizers.py. Every call here
// returns before the first HIP runtime call: invalid arguments are refused
// by validation, and crkv_plan_info / crkv_workspace_size only plan. The
// kernel launchers the library would call are not linked (see stubs below);
// reaching one is a failure.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include <hip/hip_runtime.h>

#include "crkv.h"

namespace crkv {
struct AttnArgs;
struct DecodeArgs;
struct TopkDesc;
struct SelArgs;
struct RopeArgs;
struct Q8Args;
struct CombineArgs;
struct ProbDesc;
[[noreturn]] static void launched(const char *what)
{
    std::fprintf(stderr, "host driver reached a kernel launch (%s)\n", what);
    std::abort();
}
hipError_t launch_attn_bf16_wave(int, int, const AttnArgs &, int, hipStream_t) { launched("wave"); }
hipError_t launch_attn_bf16_pair(int, int, const AttnArgs &, int, hipStream_t) { launched("pair"); }
hipError_t launch_attn_q8(int, int, const AttnArgs &, int, hipStream_t) { launched("q8 attention"); }
hipError_t launch_attn_lse(int, bool, const AttnArgs &, int, hipStream_t) { launched("pass 1"); }
hipError_t launch_attn_out_combine(int, const CombineArgs &, int, hipStream_t) { launched("output combine"); }
hipError_t launch_decode_bf16(int, const DecodeArgs &, int, int, hipStream_t) { launched("decode"); }
hipError_t launch_attn_f32(int, const AttnArgs &, int, hipStream_t) { launched("f32"); }
hipError_t launch_combine(const ProbDesc *, int, int, hipStream_t) { launched("combine"); }
hipError_t launch_topk_one(const TopkDesc &, hipStream_t) { launched("topk"); }
hipError_t launch_topk_batched(const TopkDesc *, int, hipStream_t) { launched("topk"); }
hipError_t launch_topk_inline(const TopkDesc *, int, hipStream_t) { launched("topk"); }
hipError_t launch_kvsel(bool, const SelArgs &, int, hipStream_t) { launched("kvsel"); }
hipError_t launch_rope_shift(int, bool, const RopeArgs &, int, hipStream_t) { launched("rope"); }
hipError_t launch_quantize_q8(int, const Q8Args &, int, const Q8Args &, int, hipStream_t) { launched("q8"); }
hipError_t launch_decode_q8(int, const DecodeArgs &, int, int, hipStream_t) { launched("q8 decode"); }
}  // namespace crkv

static int g_fail = 0;
#define EXPECT(cond)                                                                      \
    do {                                                                                  \
        if (!(cond)) {                                                                    \
            std::fprintf(stderr, "%s:%d: expected %s (last error: %s)\n", __FILE__, __LINE__, \
                         #cond, crkv_last_error());                                      \
            ++g_fail;                                                                     \
        }                                                                                 \
    } while (0)

static char *fake(size_t off) { return reinterpret_cast<char *>(0x10000) + off * 0x1000; }

// A problem with placeholder (aligned, never dereferenced) device addresses.
struct FakeProblem {
    std::vector<const void *> K, V;
    std::vector<int32_t> lens;
    int q_len;
    FakeProblem(const std::vector<int> &docs, int q, int gen = 0) : q_len(q)
    {
        for (size_t c = 0; c <= docs.size(); ++c) {
            const int len = c < docs.size() ? docs[c] : gen + q_len;
            lens.push_back(len);
            K.push_back(len ? fake(16 + 2 * c) : nullptr);
            V.push_back(len ? fake(17 + 2 * c) : nullptr);
        }
    }
    // the C struct, pointing into this object's own arrays
    crkv_problem c() const
    {
        crkv_problem p;
        std::memset(&p, 0, sizeof p);
        p.Q = fake(1);
        p.out = fake(2);
        p.impact = reinterpret_cast<float *>(fake(3));
        p.chunk_K = K.data();
        p.chunk_V = V.data();
        p.chunk_len = lens.data();
        p.m = (int)lens.size() - 1;
        p.q_len = q_len;
        return p;
    }
};

static crkv_opts opts(int dtype, int mode)
{
    crkv_opts o;
    crkv_opts_init(&o);
    o.dtype = dtype;
    o.mode = mode;
    return o;
}

// Plans a batch (kernel choice, row tiles, grid) and sizes its scratch.
static void plan_round_trip(const std::vector<FakeProblem *> &ps, int H, int H_kv, int d, int dtype, int mode)
{
    std::vector<crkv_problem> arr;
    for (auto *p : ps)
        arr.push_back(p->c());
    crkv_opts o = opts(dtype, mode);
    int kernel = -1, rt = -1, wg = -1;
    EXPECT(crkv_plan_info(arr.data(), (int)arr.size(), H, H_kv, d, &o, &kernel, &rt, &wg) == CRKV_OK);
    EXPECT(dtype != CRKV_F32 || kernel == 0);
    EXPECT(dtype != CRKV_BF16 || kernel == 1 || kernel == 2);
    EXPECT(dtype != CRKV_KV_Q8 || (kernel == 1 && (rt == 4 || rt == 5)));
    EXPECT(rt >= 1 && wg >= 1);
    EXPECT(crkv_workspace_size(arr.data(), (int)arr.size(), H, H_kv, d, &o) > 0);
    crkv_plan_stat st;
    EXPECT(crkv_plan_stats(arr.data(), (int)arr.size(), H, H_kv, d, &o, &st) == CRKV_OK);
    EXPECT(st.kernel == kernel && st.row_tiles == rt && st.workgroups == wg);
    EXPECT(st.scratch_bytes == crkv_workspace_size(arr.data(), (int)arr.size(), H, H_kv, d, &o));
    EXPECT(st.max_ranges >= 1 && (st.split_blocks == 0) == (st.combine_workgroups == 0));
    EXPECT(st.split_blocks == 0 || st.pass1_separate == 1);
    EXPECT(dtype == CRKV_F32 || st.model_cycles > 0);
    if (dtype == CRKV_BF16 && mode == CRKV_IMPACT_QUERY_ROWS) {
        bool q1 = true;
        for (auto *p : ps)
            q1 = q1 && p->q_len == 1;
        if (q1 && H / H_kv <= 16)
            EXPECT(crkv_decode_workspace_size(arr.data(), (int)arr.size(), H, H_kv, d, &o) > 0);
    }
}

int main()
{
    // ---------------------------------------------------------------- validation
    {
        FakeProblem p({64, 64}, 16);
        crkv_opts o = opts(CRKV_F32, CRKV_IMPACT_QUERY_ROWS);
        auto call = [&](const crkv_problem &q, int H, int H_kv, int d, const crkv_opts &oo) {
            return crkv_attn_chunks(q.Q, q.chunk_K, q.chunk_V, q.chunk_len, q.m, q.q_len, H, H_kv, d, q.out,
                                    q.impact, &oo);
        };
        crkv_problem q = p.c();
        q.Q = nullptr;
        EXPECT(call(q, 4, 4, 64, o) == CRKV_E_INVAL);
        q = p.c();
        q.impact = nullptr;
        EXPECT(call(q, 4, 4, 64, o) == CRKV_E_INVAL);
        EXPECT(call(p.c(), 6, 4, 64, o) == CRKV_E_INVAL);
        EXPECT(call(p.c(), 0, 4, 64, o) == CRKV_E_INVAL);
        EXPECT(call(p.c(), 4, 4, 96, o) == CRKV_E_UNSUPPORTED);
        q = p.c();
        q.q_len = 17;
        EXPECT(call(q, 4, 4, 64, o) == CRKV_E_INVAL);
        q = p.c();
        q.q_len = 0;
        EXPECT(call(q, 4, 4, 64, o) == CRKV_E_INVAL);
        FakeProblem neg({64, 64}, 16);
        neg.lens[1] = -3;
        EXPECT(call(neg.c(), 4, 4, 64, o) == CRKV_E_INVAL);
        FakeProblem nul({64, 64}, 16);
        nul.K[1] = nullptr;
        EXPECT(call(nul.c(), 4, 4, 64, o) == CRKV_E_INVAL);
        FakeProblem mis({64, 64}, 16);
        mis.V[0] = fake(40) + 8;
        EXPECT(call(mis.c(), 4, 4, 64, o) == CRKV_E_INVAL);
        q = p.c();
        q.Q = fake(1) + 4;
        EXPECT(call(q, 4, 4, 64, o) == CRKV_E_INVAL);
        q = p.c();
        q.impact = reinterpret_cast<float *>(fake(3) + 2);
        EXPECT(call(q, 4, 4, 64, o) == CRKV_E_INVAL);
        crkv_opts bad = o;
        bad.dtype = 7;
        EXPECT(call(p.c(), 4, 4, 64, bad) == CRKV_E_INVAL);
        bad = o;
        bad.mode = 5;
        EXPECT(call(p.c(), 4, 4, 64, bad) == CRKV_E_INVAL);
        bad = o;
        bad.workspace = fake(50) + 16;
        EXPECT(call(p.c(), 4, 4, 64, bad) == CRKV_E_INVAL);
        bad = o;
        bad.dtype = 9;
        EXPECT(call(p.c(), 4, 4, 64, bad) == CRKV_E_INVAL);
        EXPECT(crkv_attn_chunks_batched(nullptr, 0, 4, 4, 64, &o) == CRKV_E_INVAL);
        EXPECT(crkv_attn_chunks_batched(nullptr, 1, 4, 4, 64, &o) == CRKV_E_INVAL);
        // static-scratch entry point: a caller workspace, and a batch too large
        crkv_opts ws = opts(CRKV_BF16, CRKV_IMPACT_QUERY_ROWS);
        ws.workspace = fake(64);
        const crkv_problem pc = p.c();
        EXPECT(crkv_attn_chunks_batched_static(&pc, 1, 4, 4, 64, &ws) == CRKV_E_INVAL);
        std::vector<FakeProblem> big(4, FakeProblem(std::vector<int>(8, 8192), 128));
        std::vector<crkv_problem> ba;
        for (auto &b : big)
            ba.push_back(b.c());
        crkv_opts cr = opts(CRKV_BF16, CRKV_IMPACT_CROSS_DOC);
        EXPECT(crkv_attn_chunks_batched_static(ba.data(), 4, 32, 32, 128, &cr) == CRKV_E_UNSUPPORTED);
    }
    // ---------------------------------------------------------------- top-k arguments
    {
        crkv_opts o = opts(CRKV_F32, 0);
        const float *imp = reinterpret_cast<const float *>(fake(4));
        int32_t *idx = reinterpret_cast<int32_t *>(fake(5));
        EXPECT(crkv_topk(nullptr, 10, 3, idx, &o) == CRKV_E_INVAL);
        EXPECT(crkv_topk(imp, 10, 0, idx, &o) == CRKV_E_INVAL);
        EXPECT(crkv_topk(imp, 10, 11, idx, &o) == CRKV_E_INVAL);
        EXPECT(crkv_topk(imp, 100000, 9000, idx, &o) == CRKV_E_UNSUPPORTED);
        const float *ip[2] = {imp, imp};
        int32_t nn[2] = {10, 10}, kk[2] = {3, 12};
        int32_t *xp[2] = {idx, idx};
        EXPECT(crkv_topk_batched(ip, nn, kk, xp, 2, &o) == CRKV_E_INVAL);
        EXPECT(crkv_topk_batched(ip, nn, kk, xp, 0, &o) == CRKV_E_INVAL);
    }
    // ---------------------------------------------------------------- small host-only functions
    EXPECT(crkv_budget(128, 0.1) == 12 && crkv_budget(10000, 0.15) == 1500 && crkv_budget(8192, 0.05) == 409);
    EXPECT(crkv_budget(3, 0.1) == 1 && crkv_budget(-1, 0.1) == -1 && crkv_budget(10, 1.5) == -1);
    EXPECT(crkv_q8_bytes(8, 2500, 128, CRKV_Q8_K) == (size_t)8 * 2500 * 128 + 8 * 128 * 4);
    EXPECT(crkv_q8_bytes(8, 2500, 128, CRKV_Q8_V) == (size_t)8 * 2500 * 128 + 8 * 2500 * 4);
    EXPECT(crkv_q8_bytes(8, 0, 128, CRKV_Q8_K) == 0 && crkv_q8_bytes(8, 10, 96, CRKV_Q8_K) == 0);
    for (int s = 1; s >= -5; --s)
        EXPECT(crkv_status_string(s) != nullptr);
    EXPECT(crkv_version() == CRKV_VERSION);
    {
        // rope / gather / quantise argument checks
        crkv_opts o = opts(CRKV_BF16, 0);
        crkv_rope_seg rs{fake(6), 100, 3};
        EXPECT(crkv_rope_shift(&rs, 1, 8, 96, 10000.0, &o) != CRKV_OK);
        EXPECT(crkv_rope_shift(&rs, 1, 8, 128, 0.5, &o) != CRKV_OK);
        crkv_rope_seg bad_len{fake(6), -1, 3};
        EXPECT(crkv_rope_shift(&bad_len, 1, 8, 128, 10000.0, &o) != CRKV_OK);
        crkv_q8_seg qs{fake(7), fake(8), 100, 5};
        EXPECT(crkv_quantize_q8(&qs, 1, 8, 128, &o) != CRKV_OK);
        void *ck[2] = {fake(9), fake(10)}, *cv[2] = {fake(11), fake(12)};
        int32_t cl[2] = {10, -1};
        crkv_kv_select sel{ck, cv, cl, 1, reinterpret_cast<const int32_t *>(fake(13)), 4, fake(14), fake(15)};
        EXPECT(crkv_gather_kv(&sel, 1, 8, 128, &o) != CRKV_OK);
        EXPECT(crkv_scatter_kv(&sel, 1, 8, 128, &o) != CRKV_OK);
    }
    // ---------------------------------------------------------------- planner round trips
    {
        FakeProblem tiny({64, 64}, 16);
        plan_round_trip({&tiny}, 4, 4, 64, CRKV_F32, CRKV_IMPACT_QUERY_ROWS);
        FakeProblem l2({512, 512, 512, 512}, 64);
        plan_round_trip({&l2}, 32, 32, 128, CRKV_BF16, CRKV_IMPACT_QUERY_ROWS);
        std::vector<FakeProblem> l3(32, FakeProblem({2500, 2500, 2500, 2500}, 100));
        std::vector<FakeProblem *> l3p;
        for (auto &p : l3)
            l3p.push_back(&p);
        plan_round_trip(l3p, 32, 8, 128, CRKV_BF16, CRKV_IMPACT_QUERY_ROWS);
        FakeProblem cd(std::vector<int>(8, 1024), 128);
        plan_round_trip({&cd}, 32, 32, 128, CRKV_BF16, CRKV_IMPACT_CROSS_DOC);
        plan_round_trip({&cd}, 32, 32, 128, CRKV_BF16, CRKV_IMPACT_ALL_ROWS);
        plan_round_trip(l3p, 32, 8, 128, CRKV_KV_Q8, CRKV_IMPACT_QUERY_ROWS);   // 8-bit segments
        plan_round_trip({&cd}, 32, 32, 128, CRKV_KV_Q8, CRKV_IMPACT_CROSS_DOC);
        std::vector<FakeProblem> rg;
        unsigned s = 7;
        auto rnd = [&](int lo, int hi) {
            s = s * 1103515245u + 12345u;
            return lo + (int)((s >> 8) % (unsigned)(hi - lo + 1));
        };
        for (int r = 0; r < 16; ++r)
            rg.emplace_back(std::vector<int>{rnd(1024, 4096), rnd(1024, 4096), rnd(1024, 4096), rnd(1024, 4096)},
                            rnd(32, 256));
        std::vector<FakeProblem *> rgp;
        for (auto &p : rg)
            rgp.push_back(&p);
        plan_round_trip(rgp, 64, 8, 128, CRKV_BF16, CRKV_IMPACT_QUERY_ROWS);
        // edge shapes: empty and length-1 chunks, no documents, generated tokens, decode steps
        FakeProblem e1({0, 1, 0, 300}, 3);
        FakeProblem e2({}, 45);
        FakeProblem e3({511, 2}, 1, 77);
        plan_round_trip({&e1, &e2, &e3}, 8, 2, 128, CRKV_BF16, CRKV_IMPACT_QUERY_ROWS);
        plan_round_trip({&e1, &e2}, 6, 2, 64, CRKV_BF16, CRKV_IMPACT_CROSS_DOC);
        plan_round_trip({&e1, &e2, &e3}, 3, 1, 64, CRKV_F32, CRKV_IMPACT_ALL_ROWS);
        std::vector<FakeProblem> dec(32, FakeProblem({2500, 2500, 2500, 2500}, 1, 227));
        std::vector<FakeProblem *> decp;
        for (auto &p : dec)
            decp.push_back(&p);
        plan_round_trip(decp, 32, 8, 128, CRKV_BF16, CRKV_IMPACT_QUERY_ROWS);
        // every built (kernel, row tiles) choice through the planner's override
        const char *kernels[2] = {"wave", "pair"};
        const char *rts[7] = {"1", "2", "3", "4", "5", "6", "7"};
        for (const char *k : kernels)
            for (const char *r : rts) {
                setenv("CRKV_BF16_KERNEL", k, 1);
                setenv("CRKV_ROW_TILES", r, 1);
                std::vector<crkv_problem> arr;
                for (auto *p : rgp)
                    arr.push_back(p->c());
                crkv_opts o = opts(CRKV_BF16, CRKV_IMPACT_QUERY_ROWS);
                int kernel, rt, wg;
                (void)crkv_plan_info(arr.data(), (int)arr.size(), 64, 8, 128, &o, &kernel, &rt, &wg);
                (void)crkv_workspace_size(arr.data(), (int)arr.size(), 64, 8, 128, &o);
            }
        unsetenv("CRKV_BF16_KERNEL");
        unsetenv("CRKV_ROW_TILES");
        // key ranges: none, forced counts (more ranges than key tiles too), pass-1 forms
        const char *splits[4] = {"off", "2", "7", "100000"};
        for (const char *sp : splits) {
            setenv("CRKV_KEY_SPLIT", sp, 1);
            plan_round_trip(rgp, 64, 8, 128, CRKV_BF16, CRKV_IMPACT_QUERY_ROWS);
            plan_round_trip({&cd}, 32, 32, 128, CRKV_BF16, CRKV_IMPACT_CROSS_DOC);
            plan_round_trip({&e1, &e2, &e3}, 8, 2, 128, CRKV_BF16, CRKV_IMPACT_QUERY_ROWS);
            plan_round_trip(l3p, 32, 8, 128, CRKV_KV_Q8, CRKV_IMPACT_QUERY_ROWS);
        }
        unsetenv("CRKV_KEY_SPLIT");
        const char *sweeps[2] = {"fused", "split"};
        for (const char *sw : sweeps) {
            setenv("CRKV_SWEEP1", sw, 1);
            plan_round_trip(rgp, 64, 8, 128, CRKV_BF16, CRKV_IMPACT_QUERY_ROWS);
            plan_round_trip({&l2}, 32, 32, 128, CRKV_BF16, CRKV_IMPACT_QUERY_ROWS);
        }
        unsetenv("CRKV_SWEEP1");
    }
    if (g_fail) {
        std::fprintf(stderr, "%d expectations failed\n", g_fail);
        return 1;
    }
    std::printf("HOST_SANITIZE_OK\n");
    return 0;
}
