// Copies the K and V rows of selected keys between a problem's segment table
// and packed buffers, for gfx950: gather (segments -> packed) and scatter
// (packed -> segments).
//
// What it moves (CacheBlend summary, the three-phase flowchart: the K/V
// values of exactly the high-impact tokens are recomputed, and generation
// then runs on the fused cache): for every KV head h and selected key j,
//   gather:  K_sel[h][j] = K_cat[h][idx[j]]   (and V)
//   scatter: K_cat[h][idx[j]] = K_sel[h][j]   (and V)
// with K_cat the concatenation of the segments (never formed). A position
// outside [0, N) gathers a zero row and scatters nothing.
//
// Pure data movement, bound by HBM: each workgroup takes kSelKeysPerItem
// selected keys of one problem, resolves their (segment, offset) once into
// LDS, then streams every (key, head, K|V) row as 16-byte vector loads and
// stores, four in flight per thread. Rows are 128-512 bytes, so each row is
// one or more fully used 64-byte segments of a wave's request.
#include "crkv_internal.h"
#include "device_util.h"

namespace crkv {

template <bool SCATTER>
__global__ void __launch_bounds__(kSelThreads) kvsel_kernel(const SelArgs a)
{
    // Per selected key of the item: the address of its K and V rows for KV
    // head 0 and the byte stride between heads (0 marks a position outside
    // the sequence). Resolved once, so the copy loop issues no dependent
    // global loads and keeps all of its row loads in flight.
    __shared__ uint64_t s_k[kSelKeysPerItem], s_v[kSelKeysPerItem], s_hs[kSelKeysPerItem];
    const SelItem it = a.items[blockIdx.x];
    const SelProb pr = a.probs[it.prob];
    const gptr<const SelSeg> segs = as_global(pr.segs);
    const int tid = threadIdx.x;
    const int nj = min(kSelKeysPerItem, pr.k - it.j0);
    if (tid < kSelKeysPerItem) {
        uint64_t kaddr = 0, vaddr = 0, hs = 0;
        if (tid < nj) {
            const int i = as_global(pr.idx)[it.j0 + tid];
            // last segment starting at or before i (empty segments share the
            // start of the next one, so the last such one holds i if any does)
            int lo = 0, hi = pr.n_seg - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (segs[mid].start <= i)
                    lo = mid;
                else
                    hi = mid - 1;
            }
            const int start = segs[lo].start, len = segs[lo].len;
            if (i >= 0 && i >= start && i < start + len) {
                const uint64_t row = (uint64_t)(i - start) * a.row_bytes;
                kaddr = reinterpret_cast<uint64_t>(segs[lo].K) + row;
                vaddr = reinterpret_cast<uint64_t>(segs[lo].V) + row;
                hs = (uint64_t)len * a.row_bytes;
            }
        }
        s_k[tid] = kaddr;
        s_v[tid] = vaddr;
        s_hs[tid] = hs;
    }
    __syncthreads();

    const int cpr = a.row_bytes >> 4;              // 16-byte chunks per row (8, 16, 32)
    const int rows_per_pass = kSelThreads / cpr;   // rows a pass of the workgroup covers
    const int ch = tid % cpr;
    const int two_h = 2 * a.H_kv;
    const int n_rows = nj * two_h;                 // (key, head, K|V) rows of the item
    const uint64_t sel_head = (uint64_t)pr.k * a.row_bytes;
    const uint64_t sel0 = (uint64_t)it.j0 * a.row_bytes + 16 * ch;
    constexpr int kInFlight = 4;
    for (int r0 = tid / cpr; r0 < n_rows; r0 += kInFlight * rows_per_pass) {
        // Addresses first (ALU and LDS only), then every load, then every
        // store. Every load is unconditional (a lane with nothing to move
        // reads its own valid packed row and drops it), so the compiler never
        // rewrites a register that a load in flight will fill.
        uint64_t src[kInFlight], dst[kInFlight];
        bool zero[kInFlight], put[kInFlight];
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) {
            const bool live = r0 + u * rows_per_pass < n_rows;
            const int r = min(r0 + u * rows_per_pass, n_rows - 1);
            const int jj = r / two_h;
            const int rem = r - jj * two_h;
            const int h = rem >> 1;
            const bool is_v = rem & 1;
            const uint64_t cat0 = is_v ? s_v[jj] : s_k[jj];
            const uint64_t sel = reinterpret_cast<uint64_t>(is_v ? pr.V_sel : pr.K_sel) + h * sel_head + sel0 +
                                 (uint64_t)jj * a.row_bytes;
            const uint64_t cat = cat0 + h * s_hs[jj] + 16 * ch;
            // a position outside the sequence (cat0 == 0) gathers zeros and scatters nothing
            src[u] = (SCATTER || cat0 == 0) ? sel : cat;
            dst[u] = SCATTER ? cat : sel;
            zero[u] = !SCATTER && cat0 == 0;
            put[u] = live && (!SCATTER || cat0 != 0);
        }
        u32x4 buf[kInFlight];
#pragma unroll
        for (int u = 0; u < kInFlight; ++u)
            buf[u] = *as_global(reinterpret_cast<const u32x4 *>(src[u]));
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) {
            if (zero[u])
                buf[u] = u32x4{0u, 0u, 0u, 0u};
            if (put[u])
                *as_global(reinterpret_cast<u32x4 *>(dst[u])) = buf[u];
        }
    }
}

hipError_t launch_kvsel(bool scatter, const SelArgs &args, int n_items, hipStream_t stream)
{
    if (n_items <= 0)
        return hipSuccess;
    if (scatter)
        hipLaunchKernelGGL(kvsel_kernel<true>, dim3(n_items), dim3(kSelThreads), 0, stream, args);
    else
        hipLaunchKernelGGL(kvsel_kernel<false>, dim3(n_items), dim3(kSelThreads), 0, stream, args);
    return hipGetLastError();
}

}  // namespace crkv
