// Host-side launch interfaces between the C ABI (api.cpp) and the kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dattn {

// Kernel launch bracketing for per-kernel timing (api.cpp).  Between
// prof_begin and prof_end, the kernels launched on this thread carry the
// record's events: the first launch its start event, every launch its stop
// event, so the record spans the first kernel's start to the last one's end
// as the dispatches themselves report them (launch overhead excluded).
void prof_begin(const char* name, hipStream_t s);
void prof_end(hipStream_t s);
struct ProfEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
ProfEvents prof_events_for_launch();  // both null when timing is off

// Every kernel of the library is launched through here.
template <typename F, typename... Args>
void launch_kernel(F kernel, dim3 grid, dim3 block, hipStream_t s, Args... args) {
  const ProfEvents ev = prof_events_for_launch();
  hipExtLaunchKernelGGL(kernel, grid, block, 0, s, ev.start, ev.stop, 0, args...);
}

// Compute units of the current device, queried once per device (256 when the
// device cannot be queried); the decode calls make no other device queries.
int device_cu_count();

struct GqaArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* seq_lens;
  const int32_t* page_table;  // nullptr: contiguous
  int32_t window, n_sink;
  void* out;
  float* lse;
  float* part_o;    // [B*Hq, num_splits, D]  (num_splits > 1)
  float* part_lse;  // [B*Hq, num_splits]    (log2 units)
  int32_t B, Hq, Hkv, D, G;
  int32_t page_size, log2_page, max_pages, num_splits;
  int32_t bf16;
  float scale_log2;  // softmax scale * log2(e)
  // nullptr, or one sink logit per query head [Hq] (natural log): an extra
  // softmax-denominator term exp(sink) with a zero value
  const float* sink;
  // nullptr, or 16-token blocks attended besides the partial last block
  // (window and sinks are then unused):
  //   list_count == nullptr: per query head [B, Hq, list_len], ascending,
  //     -1 padded; the grid runs one query head per workgroup;
  //   else per (sequence, KV head) [B, Hkv, list_len] entries block | heads
  //     << 24 (bit h: query head h of the group attends the block), ascending,
  //     list_count[b * Hkv + kvh] of them.
  const int32_t* block_list;
  int32_t list_len;
  const int32_t* list_count;
};

hipError_t launch_gqa(const GqaArgs& a, hipStream_t s);
// Resident workgroups per CU of the split kernel for this shape (0 if unknown).
int gqa_blocks_per_cu(bool bf16, int D, int G, bool paged, int page_size);
int gqa_listed_blocks_per_cu(bool bf16, int D, int G, bool uni);

// Query-aware page selection (Quest): per-block key min/max summaries and the
// per-query-head bounds; the choice itself runs on the top-k select.
struct QuestArgs {
  const void* q;              // [B, Hq, D]
  const void* k;              // K cache, decode_attn_gqa layout
  const int32_t* seq_lens;
  const int32_t* page_table;  // or nullptr (contiguous)
  void* kminmax;              // [B, Hkv, max_blocks, 2, D] k's type
  float* upper;               // [B * Hq, max_blocks] fp32
  int32_t* n_full;            // [B * Hq]: full blocks of the row's sequence
  int32_t B, Hq, Hkv, D, G, page_size, log2_page, max_pages, max_blocks, first_block;
  int32_t bf16;
};

hipError_t launch_quest_minmax(const QuestArgs& a, hipStream_t s);
hipError_t launch_quest_bounds(const QuestArgs& a, hipStream_t s);

// Union of the chosen blocks of the G query heads of each (sequence, KV
// head): sel [B * Hq, budget] (ascending, -1 padded) -> list [B * Hkv, cap]
// entries block | heads << 24 ascending, count [B * Hkv].
struct QuestUnionArgs {
  const int32_t* sel;
  const int32_t* seq_lens;
  int32_t* list;
  int32_t* count;
  int32_t B, Hq, Hkv, G, budget, cap, max_blocks;
};
constexpr int kQuestUnionMaxBlocks = 8192;  // bitmap of 256 words per head in LDS
hipError_t launch_quest_union(const QuestUnionArgs& a, hipStream_t s);

struct CombineArgs {
  const float* part_o;    // [rows, splits, D]
  const float* part_lse;  // [rows, splits] (log2 units)
  // nullptr: part_o holds o / l and part_lse log2(sum 2^s).  Otherwise
  // part_o holds the unnormalised sum of 2^(s - m) v, part_lse the reference
  // m and part_l [rows, splits] the sum of 2^(s - m).
  const float* part_l;
  void* out;              // [rows, D]
  float* lse;             // [rows] natural log, or nullptr
  int32_t rows, splits, D;
  int32_t bf16;
  // nullptr, or a sink logit per head (natural log) for row r: sink[r % sink_heads]
  const float* sink = nullptr;
  int32_t sink_heads = 1;
  // nullptr, or the item table of a balanced MLA call ([B][2]: first item,
  // item count of sequence b): row r = b * heads + h then merges the partials
  // of rows first * heads + h * count + j, j < count.  `splits` is then the
  // item count per sequence a plan of full-length sequences makes (rows
  // r * splits + j: loaded before the table is read, and kept when it agrees).
  const int32_t* items = nullptr;
  int32_t heads = 1;
};

hipError_t launch_combine(const CombineArgs& a, hipStream_t s);

struct MlaArgs {
  const uint16_t* q;        // [B, H, Dq] bf16
  const uint16_t* latent;   // paged [pages, P, Dq] or contiguous [B, S_max, Dq]
  const int32_t* seq_lens;  // dense mode
  const int32_t* page_table;
  const int32_t* idx;       // sparse mode: [B, k_sel]
  int32_t k_sel;
  uint16_t* out;            // [B, H, Dc] (num_splits == 1)
  float* lse;
  float* part_o;             // [B, H, splits, Dc] unnormalised sums
  float* part_lse;           // [B, H, splits] reference maximum (log2 units)
  float* part_l;             // [B, H, splits] softmax denominators
  int32_t B, H, S_max, page_size, log2_page, max_pages, num_splits;
  int32_t heads_per_wg;     // 128 (four waves) or 64 (two waves) query heads per workgroup
  float scale_log2;
  // Balanced splits (flat_target > 0; dense 128-head calls over a contiguous
  // cache whose split count the library plans): every sequence is cut into
  // items of `chunk` tokens, chunk = the total tokens / flat_target rounded up
  // to whole 32-row tiles and held within [flat_min, flat_max], so that long
  // and short sequences make items of about equal work.  Sequence b's items
  // (first f, count n) write rows f * H + h * n + j; flat_table [B][2] gets
  // each sequence's f and n.  The grid holds flat_slots items (a multiple of 8, at least
  // the items any lengths within the cache can make).
  int32_t flat_target = 0, flat_min = 0, flat_max = 0, flat_slots = 0;
  int32_t* flat_table = nullptr;
};
// Sequences a balanced MLA call plans for (8 lengths per lane of one wave).
constexpr int kMlaFlatMaxB = 512;

// Tokens one MLA split may hold (its cache rows are tabled in LDS); the
// planner picks at least ceil(tokens / kMlaMaxSplitTokens) splits.
constexpr int kMlaMaxSplitTokens = 3840;
// Positions a sparse split may hold to run on the 32-row MLA kernel (its
// validity bitmap and row register per wave cover 8 tiles of 32).
constexpr int kMlaSparseTile32Tokens = 256;
// 128 query heads per workgroup when H allows it, else 64 (H % 64 == 0); a
// call may take 64 when H allows 128 (MlaArgs::heads_per_wg).
int mla_heads_per_workgroup(int H);
hipError_t launch_mla(const MlaArgs& a, hipStream_t s);
// Whether launch_mla runs the 32-row kernel (dense contiguous 128-head calls;
// sparse 128-head calls whose splits hold at most kMlaSparseTile32Tokens
// positions of a cache with S_max * 1152 < 2^32; paged 128-head calls with
// pages of at least 8 rows and at most 128 pages per split).
bool mla_uses_tile32(const MlaArgs& a);
bool mla_sparse_on_tile32(const MlaArgs& a);

struct IndexerArgs {
  const void* q;           // [B, Hi, 128] bf16 or fp8 e4m3
  const float* w;          // [B, Hi]
  const void* k;           // [B, S_max, 128], q's type
  const int32_t* seq_lens;
  float* scores;           // [B, S_max]
  int32_t B, Hi, S_max;
  int32_t tok_per_wg;      // set by the launcher
  int32_t fp8;             // 1: q and k are fp8 e4m3 (OCP e4m3fn)
  // nullptr, or the top-k workspace: when each workgroup's token range is
  // one top-k chunk, the indexer also writes each chunk's histogram of the
  // scores' top key byte (the select's first level) at hist0 + b *
  // hist_row_words + chunk * 256.  The launcher clears hist0 when the ranges
  // do not match the chunks.
  uint32_t* hist0;
  int64_t hist_row_words;
};

hipError_t launch_indexer(IndexerArgs& a, hipStream_t s);

constexpr int kTopkChunk = 2048;  // tokens per top-k workgroup

struct TopkArgs {
  const float* scores;     // [B, S_max]
  const int32_t* seq_lens;
  int32_t* idx;            // [B, k]
  int32_t B, S_max, k;
  uint32_t* ws;            // topk_workspace_bytes(B, S_max), 256-byte aligned
  int32_t n_chunks;        // set by the launcher
  int64_t row_words;       // set by the launcher
  int32_t hist0_done = 0;  // 1: the first level's chunk histograms are already in ws
};

size_t topk_workspace_bytes(int B, int S_max);
int64_t topk_row_words_of(int S_max);  // 32-bit words of one row's workspace
hipError_t launch_topk(const TopkArgs& a, hipStream_t s);

// Cache append: one new row per (sequence, head) into one or two caches laid
// out [pages, heads, page_size, row] (contiguous: pages = B, page_size = S_max).
struct KvAppendArgs {
  const void* new0;        // [B, heads, row]
  const void* new1;        // second cache's rows (V), or nullptr
  void* cache0;
  void* cache1;            // nullptr for a single cache
  const int32_t* positions;  // [B]; negative: no append
  int32_t* page_table;     // [B, max_pages] or nullptr (contiguous)
  int32_t B, heads, row_bytes, page_size, log2_page, max_pages;
  int32_t ring_pages, fixed_pages;
};

hipError_t launch_kv_append(const KvAppendArgs& a, hipStream_t s);

// Streaming-read probe (diagnostics): reads `bytes` (a multiple of 16) from
// src with `grid` workgroups, `depth` (4, 8 or 16) loads in flight per
// thread; sink holds `grid` words.
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int grid, int depth,
                              hipStream_t s);

}  // namespace dattn
