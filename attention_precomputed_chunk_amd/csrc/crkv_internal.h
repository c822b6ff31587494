// Descriptors shared by the host planner and the gfx950 kernels.
//
// A call is planned on the host into three device tables, uploaded with one
// copy: per problem (ProbDesc), per segment (SegDesc), per key tile (KTile)
// and per work item (ItemDesc). Key tiles never straddle a segment, so a tile
// has one base pointer and contiguous keys; the last tile of a segment is
// partial and its missing keys are masked.
#pragma once
#include <stdint.h>

namespace crkv {

constexpr int kWaves = 4;          // SIMDs per CU: row groups per bf16 workgroup
constexpr int kThreads = kWaves * 64;
constexpr int kKeyTile = 32;       // keys staged per LDS tile
constexpr int kRowTile = 16;       // rows per MFMA row tile
// bf16 kernels. "wave": one wave per SIMD holds every role of its row tiles
// (4 waves per workgroup). "pair": a producer and a consumer wave per SIMD
// (8 waves per workgroup). Either way a workgroup covers kWaves * rt row tiles
// of one KV head.
enum Bf16Kernel { kBf16Wave = 0, kBf16Pair = 1 };
constexpr int kWaveRowTiles[5] = {1, 2, 4, 5, 7};   // rt the wave kernels are built for
constexpr int kNumWaveRowTiles = 5;
constexpr int kWaveMaxRowTilesCross = 5;        // cross-document wave kernels: 7 would spill
constexpr int kPairRowTiles[3] = {2, 4, 6};     // rt the pair kernels are built for
constexpr int kQ8RowTiles[2] = {4, 5};          // rt of the wave kernel's 8-bit builds
// Planner cost model, SIMD cycles per 32-key step of one workgroup: a fixed
// part and a part per row tile (fitted to measurements on MI355X; the wave
// kernel's per-tile part scaled by its measured 9 % gain from the pipelined
// sweep 2 and the reference-maximum sweep 1).
constexpr int kWaveStepFixed = 1884, kWaveStepPerTile = 684;
constexpr int kPairStepFixed = 3166, kPairStepPerTile = 402;
constexpr int kRowTilesF32 = 4;    // row tiles per wave, fp32 kernels
constexpr int kTopkMaxK = 8192;    // selection buffer held in LDS

struct SegDesc {
    const void *K;      // [H_kv][len][d]
    const void *V;
    int32_t len;
    int32_t start;      // position of the segment's first key
};

// A key tile is self-contained so that a kernel can fetch its data with a
// single descriptor load: row `key` of KV head g lives at
// K + (g * seg_len + key) * d elements.
struct KTile {
    const void *K;      // segment K at the tile's first key, KV head 0
    const void *V;
    int32_t n_valid;    // keys present (<= kKeyTile)
    int32_t key0;       // global position of the tile's first key
    int32_t seg_len;    // keys in the segment (the KV-head stride in rows)
    int32_t seg_lo;     // global position of the segment's first key
};
static_assert(sizeof(KTile) == 32, "kernels read a KTile as eight dwords");

struct ProbDesc {
    const void *Q;          // [H][rows][d]
    void *out;              // [H][rows][d]
    float *partial;         // [n_slots][n_keys] impact partials
    const KTile *tiles;     // key tiles in key order
    const SegDesc *segs;    // n_seg = m + 1 segments
    const int32_t *slot_end;// per slot: keys [0, slot_end) were written
    float *impact;          // [n_keys]
    int32_t n_tiles;
    int32_t n_seg;
    int32_t n_doc;
    int32_t n_keys;
    int32_t rows;           // rows per head
    int32_t pos0;           // position of row 0 (N - q_len in query-row mode, else 0)
    int32_t n_slots;
    int32_t pad;
};

// A work item is one row block (up to kWaves * RT packed 16-row tiles of one
// (problem, KV head)) over one range of its key tiles. Without a key split a
// block is one item whose range is every key tile its last row sees; with a
// split (one-wave-kernel plans, pass 1 in attn_lse_kernel) the block's key
// tiles are cut into n_ranges consecutive ranges, pass 1 writes a partial
// (max, sum) per row and range, pass 2 of each range merges them in range
// order and, for n_ranges > 1, writes an fp32 output partial that
// attn_out_combine_kernel sums in range order.
struct ItemDesc {
    int32_t prob;
    int32_t kv_head;
    int32_t tile_begin;     // first packed 16-row tile (rows packed as (j, h) within the group)
    int32_t n_rowtiles;     // <= kWaves * row tiles per wave
    int32_t n_ktiles;       // key tiles of this item's range
    int32_t slot;           // impact partial slot within the problem (one per block)
    int32_t kt_begin;       // first key tile of the range (index into the problem's list)
    int32_t range;          // 0 .. n_ranges - 1
    int32_t n_ranges;       // ranges of the block (1: no key split)
    int32_t state;          // pass-1 states of the block: state[state + range * cap_rows + packed row]
    int32_t opart;          // output partials of the block (floats), range r at + r * cap_rows * d; -1: none
    int32_t pad;
};
static_assert(sizeof(ItemDesc) == 48, "work item layout");

struct AttnArgs {
    const ProbDesc *probs;
    const ItemDesc *items;
    int32_t H, H_kv, G;
    int32_t cross;          // 1: impact skips rows of the key's own segment
    float c_log2;           // log2(e) / sqrt(d)
    int32_t cap_rows;       // packed rows per block (kWaves * RT * 16) when pass 1 runs on its own
    float *state;           // pass-1 (max, sum) pairs per (block, range, packed row), or null: pass 1 fused
    float *opart;           // fp32 output partials of split blocks
};

// Output partials of split blocks summed in range order (attn_out_combine_kernel):
// one workgroup per (split block, 16-row tile).
struct OutCombItem {
    int32_t prob;
    int32_t kv_head;
    int32_t tile;           // packed 16-row tile
    int32_t n_ranges;
    int32_t opart;          // floats: range 0 of the tile's first row in AttnArgs::opart
    int32_t pad0, pad1, pad2;
};
static_assert(sizeof(OutCombItem) == 32, "table layout");

struct CombineArgs {
    const ProbDesc *probs;
    const OutCombItem *items;
    const float *opart;
    int32_t G;
    int32_t range_stride;   // floats between the partials of consecutive ranges (cap_rows * d)
};

// Pass 1 as its own kernel (attn_lse_kernel): kLseWaves waves per workgroup,
// two per SIMD, each holding a run of the item's row tiles.
constexpr int kLseWaves = 8;
constexpr int kLseMaxRowTilesPerWave = 4;   // items of up to 32 row tiles
constexpr int kCUs = 256;                   // MI355X compute units (the planner's makespan model)
constexpr int kMinRangeTiles = 4;           // key tiles per range at least, when blocks are split

// Decode step (q_len = 1): the keys of each (problem, KV head) are split into
// ranges of key tiles; one workgroup per range writes a partial softmax state
// (per query head of the group: running max, sum, unnormalised output row),
// and one workgroup per (problem, KV head) merges the ranges in order.
constexpr int kDecodeWaves = 4;
constexpr int kDecodeMaxGroup = 16;    // query heads per KV head (one 16-row MFMA tile)

struct DecodeItem {
    int32_t prob;
    int32_t kv_head;
    int32_t tile_begin;     // first key tile of the range (index into the problem's list)
    int32_t n_tiles;
    int32_t part;           // partial slot of the range
    int32_t pad0, pad1, pad2;
};

struct DecodePair {
    int32_t prob;
    int32_t kv_head;
    int32_t part_begin;     // the pair's ranges occupy slots [part_begin, part_begin + n_parts)
    int32_t n_parts;
};

struct DecodeArgs {
    const ProbDesc *probs;
    const DecodeItem *items;
    const DecodePair *pairs;
    float *part;            // per slot: G x (max, sum) then G x d unnormalised output
    int32_t G;
    float c_log2;           // log2(e) / sqrt(d)
    int32_t H_kv;           // 8-bit segments: the scales follow H_kv * len * d code bytes
    int32_t pad;
};

struct TopkDesc {
    const float *value;
    int32_t *idx;
    int32_t n, k;
};

// Batches of up to kTopkInline top-k problems pass their descriptors as
// kernel arguments (no table upload).
constexpr int kTopkInline = 64;
struct TopkInline {
    TopkDesc d[kTopkInline];
};

// ---------------------------------------------------------------- selected-key K/V gather / scatter
constexpr int kSelKeysPerItem = 16;   // selected keys per workgroup
constexpr int kSelThreads = 256;

struct SelSeg {               // one segment of a problem's table
    const void *K;            // [H_kv][len][d]
    const void *V;
    int32_t start;            // position of its first key in the concatenation
    int32_t len;
    int32_t pad0, pad1;
};

struct SelProb {
    const SelSeg *segs;       // n_seg = m + 1 segments, in key order
    const int32_t *idx;       // [k] selected positions
    void *K_sel;              // [H_kv][k][d]
    void *V_sel;
    int32_t n_seg;
    int32_t k;
    int32_t pad0, pad1;
};

struct SelItem {              // keys j0 .. j0 + kSelKeysPerItem - 1 of one problem
    int32_t prob;
    int32_t j0;
};

struct SelArgs {
    const SelProb *probs;
    const SelItem *items;
    int32_t H_kv;
    int32_t row_bytes;        // d * element size: 128, 256 or 512
};
static_assert(sizeof(SelSeg) == 32 && sizeof(SelProb) == 48 && sizeof(SelItem) == 8, "table layout");

// ---------------------------------------------------------------- key re-positioning (rotary embedding)
constexpr int kRopeThreads = 256;
constexpr int kRopeRowsPerItem = 256;   // rows ([H_kv * len] of a segment) per workgroup

struct RopeSeg {
    void *K;                  // [H_kv][len][d], rotated in place
    const float *cs;          // cos of the d/2 angles, then their sin
    int32_t rows;             // H_kv * len
    int32_t pad;
};

struct RopeItem {
    int32_t seg;
    int32_t row0;
};

struct RopeArgs {
    const RopeSeg *segs;
    const RopeItem *items;
    int32_t d;
    int32_t bf16;
};
static_assert(sizeof(RopeSeg) == 24 && sizeof(RopeItem) == 8, "table layout");

// ---------------------------------------------------------------- 8-bit K/V segments
// A segment [H_kv][len][d] in the 8-bit format is one buffer: int8 codes
// [H_kv][len][d], then float32 scales (value = code * scale): [H_kv][d], one
// per channel over the segment's tokens, for K; [H_kv][len], one per token,
// for V.
constexpr int kQ8Threads = 256;
constexpr int kQ8RowsPerItem = 256;     // V: rows ([H_kv * len] of a segment) per workgroup

struct Q8Seg {
    const void *x;            // bf16 [H_kv][len][d]
    void *q8;                 // codes, then scales
    int32_t rows;             // H_kv * len
    int32_t len;
};

struct Q8Item {
    int32_t seg;
    int32_t row0;             // V: first row of the workgroup; K: the KV head
};

struct Q8Args {
    const Q8Seg *segs;
    const Q8Item *items;
};
static_assert(sizeof(Q8Seg) == 24 && sizeof(Q8Item) == 8, "table layout");

}  // namespace crkv
