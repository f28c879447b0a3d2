// C ABI of the dattn library: argument validation, split planning, workspace
// carving and kernel launches on the caller's stream.  See include/dattn.h.
#include "../../include/dattn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "internal.hpp"

namespace {

constexpr int kMaxSplits = 64;
constexpr int kMlaMaxSplits = 256;
constexpr int kTopkMax = 16384;
constexpr int kTopkMaxRow = 1 << 30;  // tokens per row the top-k indexes
thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return DATTN_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(DATTN_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool pow2(int32_t x) { return x > 0 && (x & (x - 1)) == 0; }
int ilog2(int32_t x) {
  int r = 0;
  while ((1 << r) < x) ++r;
  return r;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// ---------------------------------------------------------------- profiling
struct ProfRec {
  const char* name;
  hipEvent_t start, stop;
  bool launched;  // a kernel carried the events (else they were never recorded)
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRec> g_recs;
std::vector<hipEvent_t> g_pool;

hipEvent_t pool_get() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  // timing events without the system-scope cache flush a default event
  // performs: less added time around the kernel they bracket
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return e;
}

// ---------------------------------------------------------------- planning
// Token splits per (sequence, KV head): at most one per 256 attended tokens
// (the cap), and within that the grid is sized to one full round of resident
// workgroups (`slots` = workgroups per CU x CUs) -- a second, partial round
// only adds a tail.
int64_t gqa_split_cap(int64_t max_tokens) {
  int64_t cap = (max_tokens + 255) / 256;
  if (cap < 1) cap = 1;
  return cap < kMaxSplits ? cap : kMaxSplits;
}

int plan_gqa_splits(int32_t B, int32_t Hkv, int64_t max_tokens, int32_t req, int64_t slots) {
  if (req > 0) return req < kMaxSplits ? req : kMaxSplits;
  const int64_t units = (int64_t)B * Hkv;
  int64_t n = slots / units;
  const int64_t cap = gqa_split_cap(max_tokens);
  if (n > cap) n = cap;
  return n < 1 ? 1 : (int)n;
}

// Split-kernel workgroups to keep resident on the current device: what the
// occupancy allows, at most 4 per CU (four waves per SIMD; a fifth bought
// nothing on the GQA layer, 8 splits 86.1 us against 10 splits 87.4 us);
// 3 per CU on 256 CUs when the device cannot be queried.  Eight heads per
// KV head (a full register file: three waves per SIMD fit) run best at two
// per CU: 64 q / 8 KV heads, 16 x 8192 tokens, D128, 90.7 us at 4 splits
// against 92.3 us at 6; D64 and 16384 tokens, 93.1 against 95.5 us.
constexpr int kMaxSplitWgPerCu = 4;
int64_t gqa_slots(bool bf16, int D, int G, bool paged, int page_size) {
  const int cus = dattn::device_cu_count();
  int per = dattn::gqa_blocks_per_cu(bf16, D, G, paged, page_size);
  if (per < 1) per = 3;
  if (per > kMaxSplitWgPerCu) per = kMaxSplitWgPerCu;
  if (G >= 8 && per > 2) per = 2;
  return (int64_t)per * cus;
}

// MLA workgroups (hpw = 128 or 64 heads each, up to 160 KB of LDS) run one
// per CU: aim for at most one round of them (the count rounded down: 258
// workgroups on 256 CUs, 6 x 128 heads x 16384 tokens, took 73.5 us per
// call against 52.1 us for 222), with splits of at least min_tokens tokens.
// Dense calls take 320: below that each workgroup's 256 KB of partials and
// their combine cost more than the extra workgroups buy (128 heads x 16384
// tokens, 1 / 2 / 4 sequences: 36.2 / 39.2 / 43.8 us per call against
// 40.3 / 43.5 / 48.6 us with 128-token splits).  A split holds at most
// kMlaMaxSplitTokens tokens, which sets a floor on the count (a request
// below it is raised).  0 when the count would exceed kMlaMaxSplits.
constexpr int kMlaDenseMinSplitTokens = 320;
int plan_mla_splits(int32_t B, int32_t H, int hpw, int64_t max_tokens, int32_t req, int min_tokens) {
  const int64_t floor_n = (max_tokens + dattn::kMlaMaxSplitTokens - 1) / dattn::kMlaMaxSplitTokens;
  int64_t n;
  if (req > 0) {
    n = req;
  } else {
    const int64_t units = (int64_t)B * (H / hpw);
    const int64_t want = std::max<int64_t>(1, dattn::device_cu_count() / units);
    const int64_t cap = (max_tokens + min_tokens - 1) / min_tokens;
    n = want < cap ? want : cap;
  }
  if (n < floor_n) n = floor_n;
  if (n < 1) n = 1;
  if (n > kMlaMaxSplits) n = req > 0 ? kMlaMaxSplits : 0;
  if (n < floor_n) return 0;
  return (int)n;
}

// Splits and heads per workgroup of an MLA call.  A sparse call (a gathered
// list of k rows per sequence) whose 128-head workgroups would leave CUs idle
// takes 64-head workgroups instead: twice the workgroups, each with half the
// query fragments and half the partials to write, the second of a pair
// reading its rows from L2.  8 sequences x 2048 of 65536 rows, 128 heads,
// 16 splits: 27.0 us against 29.4 us.
struct MlaPlan {
  int splits, heads_per_wg;
};
MlaPlan plan_mla(int32_t B, int32_t H, int64_t max_tokens, int32_t req, bool sparse) {
  MlaPlan p{0, dattn::mla_heads_per_workgroup(H)};
  // A sparse call with 128-head workgroups runs on the 32-row kernel when its
  // splits hold at most kMlaSparseTile32Tokens positions: aim for one round of
  // 256 workgroups with at least two 32-row tiles per split.
  if (sparse && p.heads_per_wg == 128 && req == 0) {
    const int64_t units = (int64_t)B * (H / 128);
    const int64_t floor_n = (max_tokens + dattn::kMlaSparseTile32Tokens - 1) / dattn::kMlaSparseTile32Tokens;
    int64_t n = std::max<int64_t>(1, dattn::device_cu_count() / units);
    const int64_t cap = (max_tokens + 127) / 128;
    if (n > cap) n = cap;
    if (n < floor_n) n = floor_n;
    if (n < 1) n = 1;
    if (n <= kMlaMaxSplits) return MlaPlan{(int)n, 128};
  }
  const int min_tokens = sparse ? 128 : kMlaDenseMinSplitTokens;
  p.splits = plan_mla_splits(B, H, p.heads_per_wg, max_tokens, req, min_tokens);
  if (sparse && p.heads_per_wg == 128 && p.splits > 0 &&
      (int64_t)B * (H / 128) * p.splits < dattn::device_cu_count()) {
    const int s64 = plan_mla_splits(B, H, 64, max_tokens, req, min_tokens);
    if (s64 > 0) p = MlaPlan{s64, 64};
  }
  return p;
}

// MLA partials: unnormalised O [rows, splits, 512], reference maxima and
// denominators [rows, splits] each.
size_t mla_workspace(int64_t rows, int splits) {
  return align256((size_t)rows * splits * 512 * sizeof(float)) +
         2 * align256((size_t)rows * splits * sizeof(float));
}

// Balanced splits for a dense call whose split count the library plans
// (MlaArgs::flat_target): 128-head workgroups on the 32-row kernel over a
// contiguous cache, at most kMlaFlatMaxB sequences.  Items aim at one per CU
// and head block, of at least kMlaDenseMinSplitTokens tokens.  With one
// sequence several times longer than the rest, equal split counts per
// sequence left most CUs idle while its splits ran.  Paged calls keep the
// split grid: the paged kernel with balanced placement spilled registers and
// ran 12 % slower on a uniform batch (150.4 against 133.4 us, 64-row pages).
struct MlaFlat {
  int target = 0, slots = 0;
};
MlaFlat plan_mla_flat(int32_t B, int32_t H, int64_t cap, int32_t req, bool paged) {
  MlaFlat f;
  if (req != 0 || B > dattn::kMlaFlatMaxB || H % 128 != 0 || paged) return f;
  const int64_t target = std::max<int64_t>(1, dattn::device_cu_count() / (H / 128));
  const int64_t by_cap = (B * cap + dattn::kMlaMaxSplitTokens - 1) / dattn::kMlaMaxSplitTokens;
  const int64_t slots = (std::max(target, by_cap) + B + 7) / 8 * 8;
  if (slots * H > (int64_t(1) << 31) / 512) return f;
  f.target = (int)target;
  f.slots = (int)slots;
  return f;
}

// Items per sequence of a balanced plan when every sequence holds `cap`
// tokens: the same chunk search as the kernel's, on the host.  The combine
// loads those rows first (the split grid's layout) and keeps them when the
// item table agrees.
int mla_flat_full_items(int32_t B, int64_t cap, int target, int min_tok, int max_tok) {
  constexpr int kTile = 32;
  const int64_t tot = (int64_t)B * cap;
  int chunk = (int)std::max<int64_t>((tot + target - 1) / target, min_tok);
  chunk = std::min((chunk + kTile - 1) / kTile * kTile, max_tok);
  auto per_of = [&](int c) { return (int)((cap + c - 1) / c); };
  int items = B * per_of(chunk);
  for (int it = 0; it < 8 && items > target && chunk < max_tok; ++it) {
    const int grow = std::max(kTile, (int)((int64_t)chunk * (items - target) / target));
    chunk = std::min((chunk + grow + kTile - 1) / kTile * kTile, max_tok);
    items = B * per_of(chunk);
  }
  return per_of(chunk);
}

// [partials of slots * H rows | item table B x 2]
size_t mla_flat_workspace(const MlaFlat& f, int32_t B, int32_t H) {
  return mla_workspace((int64_t)f.slots * H, 1) + align256((size_t)B * 2 * sizeof(int32_t));
}

// Upper bound on the tokens one sequence attends: the cache capacity
// page_size * max_pages (contiguous: max_pages = 1), cut by window + sinks.
int64_t gqa_max_tokens(int32_t page_size, int32_t max_pages, int32_t window, int32_t n_sink) {
  int64_t cap = (int64_t)page_size * (max_pages < 1 ? 1 : max_pages);
  if (window > 0 && (int64_t)window + n_sink < cap) cap = (int64_t)window + n_sink;
  return cap;
}

size_t split_workspace(int64_t rows, int splits, int D) {
  if (splits <= 1) return 0;
  return align256((size_t)rows * splits * D * sizeof(float)) +
         align256((size_t)rows * splits * sizeof(float));
}

}  // namespace

namespace dattn {

int device_cu_count() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];  // 0: not queried yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < kMaxDevices) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;
  if (dev < kMaxDevices) cached[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

namespace {
// The record the launches on this thread bind to (between prof_begin and
// prof_end), and whether one of them took its start event yet.
thread_local ProfRec* tl_open = nullptr;
thread_local size_t tl_open_index = 0;
thread_local bool tl_started = false;
}  // namespace

void prof_begin(const char* name, hipStream_t s) {
  (void)s;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  tl_open = nullptr;
  if (!g_prof_on) return;
  hipEvent_t a = pool_get(), b = pool_get();
  if (!a || !b) {
    if (a) g_pool.push_back(a);
    if (b) g_pool.push_back(b);
    return;
  }
  g_recs.push_back({name, a, b, false});
  tl_open_index = g_recs.size() - 1;
  tl_open = &g_recs.back();
  tl_started = false;
}

ProfEvents prof_events_for_launch() {
  ProfEvents ev;
  if (!tl_open) return ev;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (tl_open_index >= g_recs.size()) return ev;  // records dropped meanwhile
  ProfRec& r = g_recs[tl_open_index];
  if (!tl_started) ev.start = r.start;
  ev.stop = r.stop;
  tl_started = true;
  r.launched = true;
  return ev;
}

void prof_end(hipStream_t s) {
  (void)s;
  if (!tl_open) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  // a group that launched nothing leaves no record
  if (tl_open_index + 1 == g_recs.size() && !g_recs.back().launched) {  // (else dropped meanwhile)
    g_pool.push_back(g_recs.back().start);
    g_pool.push_back(g_recs.back().stop);
    g_recs.pop_back();
  }
  tl_open = nullptr;
}

}  // namespace dattn

namespace {

template <typename F>
int launch(const char* name, hipStream_t s, F&& f) {
  dattn::prof_begin(name, s);
  hipError_t e = f();
  dattn::prof_end(s);
  if (e != hipSuccess) return hip_fail(e, name);
  return DATTN_OK;
}

// Kernels move data in 16-byte vectors.
bool aligned16(const void* p) { return (uintptr_t)p % 16 == 0; }

int check_workspace(void* ws, size_t have, size_t need) {
  if (need == 0) return DATTN_OK;
  if (!ws) return fail(DATTN_EWORKSPACE, "workspace is NULL but %zu bytes are needed", need);
  if (have < need)
    return fail(DATTN_EWORKSPACE, "workspace has %zu bytes, %zu are needed", have, need);
  if ((uintptr_t)ws % 256 != 0) return fail(DATTN_EWORKSPACE, "workspace must be 256-byte aligned");
  return DATTN_OK;
}

// ------------------------------------------------------------ debug checks
// DATTN_DEBUG=1 in the environment (or dattn_debug_enable(1)) makes the
// entry points copy the device-resident seq_lens and page_table to the host,
// synchronously on the call's stream, and check them against the layout
// contract before launching; a violation returns DATTN_EINVAL naming the
// first bad entry.  Off by default: it synchronises, so it does not suit
// stream capture or latency-sensitive loops.
std::atomic<int> g_debug{-1};  // -1: not read from the environment yet

bool debug_on() {
  int d = g_debug.load(std::memory_order_relaxed);
  if (d < 0) {
    const char* e = getenv("DATTN_DEBUG");
    d = (e && *e && strcmp(e, "0") != 0) ? 1 : 0;
    int expect = -1;
    g_debug.compare_exchange_strong(expect, d);
    d = g_debug.load(std::memory_order_relaxed);
  }
  return d > 0;
}

// The table contract on host copies (see dattn_check_tables in dattn.h).
int check_tables_host(const char* fn, const int32_t* lens, const int32_t* pt, int32_t B,
                      int32_t page_size, int32_t max_pages, int64_t num_pages) {
  const int64_t cap = (int64_t)page_size * (pt ? max_pages : 1);
  for (int32_t b = 0; b < B; ++b) {
    const int64_t L = lens[b];
    if (L < 0 || L > cap)
      return fail(DATTN_EINVAL, "%s: seq_lens[%d] = %lld outside [0, %lld]", fn, b, (long long)L,
                  (long long)cap);
    if (!pt) continue;
    const int64_t used = (L + page_size - 1) / page_size;
    for (int64_t j = 0; j < used; ++j) {
      const int64_t e = pt[(int64_t)b * max_pages + j];
      if (e < 0 || (num_pages >= 0 && e >= num_pages))
        return fail(DATTN_EINVAL, "%s: page_table[%d][%lld] = %lld names no page of the cache (%lld pages)",
                    fn, b, (long long)j, (long long)e, (long long)num_pages);
    }
  }
  return DATTN_OK;
}

// Whole pages of page_bytes from p to the end of its device allocation, or
// -1 when the allocation cannot be queried.
int64_t pages_in_allocation(const void* p, int64_t page_bytes) {
  hipDeviceptr_t base = nullptr;
  size_t size = 0;
  if (!p || page_bytes <= 0 || hipMemGetAddressRange(&base, &size, (hipDeviceptr_t)p) != hipSuccess) {
    (void)hipGetLastError();
    return -1;
  }
  const int64_t left = (int64_t)((const char*)base + size - (const char*)p);
  return left < 0 ? 0 : left / page_bytes;
}

// Copies the tables to the host on stream s and checks them.  caches: the
// device buffers the table indexes, each holding pages of page_bytes.
int debug_check(const char* fn, const int32_t* d_lens, const int32_t* d_pt, int32_t B,
                int32_t page_size, int32_t max_pages, const void* const* caches, int n_caches,
                int64_t page_bytes, hipStream_t s) {
  std::vector<int32_t> lens(B), pt;
  hipError_t e = hipMemcpyAsync(lens.data(), d_lens, sizeof(int32_t) * B, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess && d_pt) {
    pt.resize((size_t)B * max_pages);
    e = hipMemcpyAsync(pt.data(), d_pt, sizeof(int32_t) * pt.size(), hipMemcpyDeviceToHost, s);
  }
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, fn);
  int64_t num_pages = -1;
  if (d_pt) {
    for (int i = 0; i < n_caches; ++i) {
      const int64_t n = pages_in_allocation(caches[i], page_bytes);
      if (n >= 0 && (num_pages < 0 || n < num_pages)) num_pages = n;
    }
  }
  return check_tables_host(fn, lens.data(), d_pt ? pt.data() : nullptr, B, page_size, max_pages,
                           num_pages);
}

int validate_gqa(const void* q, const void* k, const void* v, const int32_t* seq_lens,
                 const int32_t* page_table, int32_t n_sink, const void* out, int32_t B,
                 int32_t Hq, int32_t Hkv, int32_t D, int32_t page_size, int32_t max_pages,
                 int32_t dtype, float scale, int32_t num_splits) {
  if (!q || !k || !v || !seq_lens || !out) return fail(DATTN_EINVAL, "decode_attn_gqa: NULL pointer argument");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(DATTN_EINVAL, "decode_attn_gqa: q, k_cache, v_cache and out must be 16-byte aligned");
  if (B < 1 || Hq < 1 || Hkv < 1) return fail(DATTN_EINVAL, "decode_attn_gqa: B, Hq, Hkv must be >= 1");
  if (B > 65535 || Hkv > 65535) return fail(DATTN_EINVAL, "decode_attn_gqa: B and Hkv must be <= 65535");
  if (Hq % Hkv != 0) return fail(DATTN_EINVAL, "decode_attn_gqa: Hq (%d) is not a multiple of Hkv (%d)", Hq, Hkv);
  const int G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(DATTN_EUNSUPPORTED, "decode_attn_gqa: group size Hq/Hkv = %d not in {1,2,4,8}", G);
  if (D != 64 && D != 128) return fail(DATTN_EUNSUPPORTED, "decode_attn_gqa: head dim %d not in {64,128}", D);
  if (dtype != DATTN_F32 && dtype != DATTN_BF16) return fail(DATTN_EUNSUPPORTED, "decode_attn_gqa: dtype %d", dtype);
  if (page_size < 1) return fail(DATTN_EINVAL, "decode_attn_gqa: page_size must be >= 1");
  if (page_table) {
    if (!pow2(page_size)) return fail(DATTN_EUNSUPPORTED, "decode_attn_gqa: paged cache needs a power-of-two page_size, got %d", page_size);
    if (max_pages < 1) return fail(DATTN_EINVAL, "decode_attn_gqa: max_pages must be >= 1");
  }
  if (n_sink < 0) return fail(DATTN_EINVAL, "decode_attn_gqa: n_sink must be >= 0");
  if (num_splits < 0) return fail(DATTN_EINVAL, "decode_attn_gqa: num_splits must be >= 0");
  if (std::isnan(scale) || std::isinf(scale)) return fail(DATTN_EINVAL, "decode_attn_gqa: scale is not finite");
  return DATTN_OK;
}

int validate_mla_common(const char* fn, const void* q, const void* latent, const void* out, int32_t B,
                        int32_t H, int32_t d_latent, int32_t d_rope, int32_t S_max, int32_t dtype,
                        float scale, int32_t num_splits) {
  if (!q || !latent || !out) return fail(DATTN_EINVAL, "%s: NULL pointer argument", fn);
  if (!aligned16(q) || !aligned16(latent) || !aligned16(out))
    return fail(DATTN_EINVAL, "%s: q, latent_cache and out must be 16-byte aligned", fn);
  if (B < 1 || H < 1 || S_max < 1) return fail(DATTN_EINVAL, "%s: B, H, S_max must be >= 1", fn);
  if (B > 65535) return fail(DATTN_EINVAL, "%s: B must be <= 65535", fn);
  if (d_latent != 512 || d_rope != 64)
    return fail(DATTN_EUNSUPPORTED, "%s: latent %d + rope %d; only 512 + 64 is built", fn, d_latent, d_rope);
  if (H % 64 != 0) return fail(DATTN_EUNSUPPORTED, "%s: H = %d is not a multiple of 64", fn, H);
  if ((int64_t)B * S_max >= ((int64_t)1 << 31))
    return fail(DATTN_EUNSUPPORTED, "%s: B * S_max must be below 2^31 cache rows", fn);
  if (H / 64 > 65535) return fail(DATTN_EINVAL, "%s: H too large", fn);
  if (dtype != DATTN_BF16) return fail(DATTN_EUNSUPPORTED, "%s: only bf16 is built", fn);
  if (num_splits < 0) return fail(DATTN_EINVAL, "%s: num_splits must be >= 0", fn);
  if (std::isnan(scale) || std::isinf(scale)) return fail(DATTN_EINVAL, "%s: scale is not finite", fn);
  return DATTN_OK;
}

// ---------------------------------------------------- allocation-free scratch
// Device memory of decode_attn_gqa_noalloc: the split partials live in this
// file-scope array instead of a caller workspace.  Each GPU the library runs
// on holds its own copy until the process ends.  In host code the name is
// only a stand-in: kernels get the address hipGetSymbolAddress returns for
// the current device, looked up once per device.
constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

int scratch_address(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "decode_attn_gqa_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(DATTN_EUNSUPPORTED, "decode_attn_gqa_noalloc: device %d", dev);
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return hip_fail(e, "decode_attn_gqa_noalloc: hipGetSymbolAddress");
    addr[dev] = p;
  }
  *out = addr[dev];
  return DATTN_OK;
}

// Steps a1-a5 (and the sink logit of N2) for decode_attn_gqa(_sink) and, with
// from_scratch, for decode_attn_gqa_noalloc: workspace is then the scratch
// array (kScratchBytes); an automatic split count is lowered until its
// partials fit, a requested one that does not fit is refused.
int run_gqa(const char* fn, const void* q, const void* k_cache, const void* v_cache, const int32_t* seq_lens,
            const int32_t* page_table, int32_t window, int32_t n_sink, const float* sink_logits, void* out,
            float* lse, int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t page_size, int32_t max_pages,
            int32_t dtype, float scale, int32_t num_splits, void* workspace, size_t workspace_bytes,
            hipStream_t s, bool from_scratch) {
  int rc = validate_gqa(q, k_cache, v_cache, seq_lens, page_table, n_sink, out, B, Hq, Hkv, D,
                        page_size, max_pages, dtype, scale, num_splits);
  if (rc) return rc;
  const bool paged = page_table != nullptr;
  int splits = plan_gqa_splits(
      B, Hkv, gqa_max_tokens(page_size, paged ? max_pages : 1, window, n_sink), num_splits,
      num_splits > 0 ? 0 : gqa_slots(dtype == DATTN_BF16, D, Hq / Hkv, paged, page_size));
  size_t need = split_workspace((int64_t)B * Hq, splits, D);
  if (from_scratch && need > workspace_bytes) {
    if (num_splits > 0)
      return fail(DATTN_EWORKSPACE, "%s: %d splits need %zu bytes of partials, above the %zu-byte scratch", fn,
                  splits, need, workspace_bytes);
    while (splits > 1 && split_workspace((int64_t)B * Hq, splits, D) > workspace_bytes) --splits;
    need = split_workspace((int64_t)B * Hq, splits, D);
  }
  if ((rc = check_workspace(workspace, workspace_bytes, need))) return rc;
  if (debug_on()) {
    const void* caches[] = {k_cache, v_cache};
    const int64_t pb = (int64_t)Hkv * page_size * D * (dtype == DATTN_BF16 ? 2 : 4);
    if ((rc = debug_check(fn, seq_lens, page_table, B, page_size, paged ? max_pages : 1, caches, 2, pb, s)))
      return rc;
  }

  dattn::GqaArgs a{};
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.seq_lens = seq_lens;
  a.page_table = page_table;
  a.window = window;
  a.n_sink = n_sink;
  a.out = out;
  a.lse = lse;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = D;
  a.G = Hq / Hkv;
  a.page_size = page_size;
  a.log2_page = paged ? ilog2(page_size) : 0;
  a.max_pages = paged ? max_pages : 1;
  a.num_splits = splits;
  a.bf16 = dtype == DATTN_BF16;
  const float sc = scale > 0.f ? scale : 1.0f / std::sqrt((float)D);
  a.scale_log2 = sc * 1.4426950408889634f;
  a.sink = sink_logits;
  if (splits > 1) {
    a.part_o = (float*)workspace;
    a.part_lse = (float*)((char*)workspace + align256((size_t)B * Hq * splits * D * sizeof(float)));
  }
  if ((rc = launch("gqa_split", s, [&] { return dattn::launch_gqa(a, s); }))) return rc;
  if (splits > 1) {
    dattn::CombineArgs c{a.part_o, a.part_lse, nullptr, out, lse, B * Hq, splits, D, a.bf16,
                         sink_logits, Hq};
    if ((rc = launch("lse_combine", s, [&] { return dattn::launch_combine(c, s); }))) return rc;
  }
  return ok();
}

}  // namespace

extern "C" {

const char* dattn_last_error(void) { return g_err.c_str(); }

int32_t dattn_version(void) { return 1; }

int dattn_stream_read_probe(const void* src, size_t bytes, uint32_t* sink, int32_t grid, int32_t depth,
                            void* stream) {
  if (!src || !sink) return fail(DATTN_EINVAL, "dattn_stream_read_probe: NULL pointer argument");
  if (!aligned16(src) || bytes % 16 != 0)
    return fail(DATTN_EINVAL, "dattn_stream_read_probe: src must be 16-byte aligned and bytes a multiple of 16");
  if (grid < 1 || grid > (1 << 20)) return fail(DATTN_EINVAL, "dattn_stream_read_probe: grid %d", grid);
  if (depth != 4 && depth != 8 && depth != 16)
    return fail(DATTN_EINVAL, "dattn_stream_read_probe: depth %d not in {4, 8, 16}", depth);
  hipStream_t s = (hipStream_t)stream;
  const int rc = launch("stream_read", s, [&] { return dattn::launch_stream_read(src, bytes, sink, grid, depth, s); });
  return rc ? rc : ok();
}

int dattn_debug_enable(int32_t on) {
  g_debug.store(on ? 1 : 0, std::memory_order_relaxed);
  return ok();
}

int dattn_check_tables(const int32_t* seq_lens, const int32_t* page_table, int32_t B,
                       int32_t page_size, int32_t max_pages, int64_t num_pages) {
  if (!seq_lens) return fail(DATTN_EINVAL, "dattn_check_tables: seq_lens is NULL");
  if (B < 1 || page_size < 1) return fail(DATTN_EINVAL, "dattn_check_tables: B and page_size must be >= 1");
  if (page_table && max_pages < 1) return fail(DATTN_EINVAL, "dattn_check_tables: max_pages must be >= 1");
  const int rc = check_tables_host("dattn_check_tables", seq_lens, page_table, B, page_size, max_pages,
                                   num_pages);
  return rc ? rc : ok();
}

int dattn_profile_enable(int32_t on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_on = on != 0;
  return ok();
}

int dattn_profile_reset(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (auto& r : g_recs) {
    if (r.start) g_pool.push_back(r.start);
    if (r.stop) g_pool.push_back(r.stop);
  }
  g_recs.clear();
  return ok();
}

int dattn_profile_read(const char* name, double* total_ms, int64_t* count) {
  if (!total_ms || !count) return fail(DATTN_EINVAL, "dattn_profile_read: NULL output");
  std::lock_guard<std::mutex> lk(g_prof_mu);
  double tot = 0.0;
  int64_t n = 0;
  for (auto& r : g_recs) {
    if (!r.launched || (name && !strstr(r.name, name))) continue;
    hipError_t e = hipEventSynchronize(r.stop);
    if (e != hipSuccess) return hip_fail(e, "dattn_profile_read");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, r.start, r.stop);
    if (e != hipSuccess) return hip_fail(e, "dattn_profile_read");
    tot += ms;
    ++n;
  }
  *total_ms = tot;
  *count = n;
  return ok();
}

// ------------------------------------------------------------------- GQA

size_t decode_attn_gqa_workspace(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t page_size,
                                 int32_t max_pages, int32_t window, int32_t n_sink,
                                 int32_t num_splits) {
  if (B < 1 || Hq < 1 || Hkv < 1 || D < 1 || page_size < 1 || num_splits < 0) return 0;
  // an upper bound on any plan: the requested count, else the split cap
  const int splits = num_splits > 0 ? (num_splits < kMaxSplits ? num_splits : kMaxSplits)
                                    : (int)gqa_split_cap(gqa_max_tokens(page_size, max_pages,
                                                                        window, n_sink));
  return split_workspace((int64_t)B * Hq, splits, D);
}

int decode_attn_gqa(const void* q, const void* k_cache, const void* v_cache, const int32_t* seq_lens,
                    const int32_t* page_table, int32_t window, int32_t n_sink, void* out, float* lse,
                    int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t page_size, int32_t max_pages,
                    int32_t dtype, float scale, int32_t num_splits, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return decode_attn_gqa_sink(q, k_cache, v_cache, seq_lens, page_table, window, n_sink, nullptr, out,
                              lse, B, Hq, Hkv, D, page_size, max_pages, dtype, scale, num_splits,
                              workspace, workspace_bytes, stream);
}

int decode_attn_gqa_sink(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* seq_lens, const int32_t* page_table, int32_t window,
                         int32_t n_sink, const float* sink_logits, void* out, float* lse, int32_t B,
                         int32_t Hq, int32_t Hkv, int32_t D, int32_t page_size, int32_t max_pages,
                         int32_t dtype, float scale, int32_t num_splits, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return run_gqa("decode_attn_gqa", q, k_cache, v_cache, seq_lens, page_table, window, n_sink, sink_logits,
                 out, lse, B, Hq, Hkv, D, page_size, max_pages, dtype, scale, num_splits, workspace,
                 workspace_bytes, (hipStream_t)stream, false);
}

int decode_attn_gqa_noalloc(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* seq_lens, const int32_t* page_table, int32_t window,
                            int32_t n_sink, const float* sink_logits, void* out, float* lse, int32_t B,
                            int32_t Hq, int32_t Hkv, int32_t D, int32_t page_size, int32_t max_pages,
                            int32_t dtype, float scale, int32_t num_splits, void* stream) {
  void* ws = nullptr;
  const int rc = scratch_address(&ws);
  if (rc) return rc;
  return run_gqa("decode_attn_gqa_noalloc", q, k_cache, v_cache, seq_lens, page_table, window, n_sink,
                 sink_logits, out, lse, B, Hq, Hkv, D, page_size, max_pages, dtype, scale, num_splits, ws,
                 kScratchBytes, (hipStream_t)stream, true);
}

// ------------------------------------------------------------------- MLA

size_t decode_attn_mla_workspace(int32_t B, int32_t H, int32_t d_latent, int32_t S_max,
                                 int32_t num_splits) {
  if (B < 1 || H < 64 || H % 64 != 0 || d_latent < 1 || S_max < 1 || num_splits < 0) return 0;
  const int splits = plan_mla(B, H, S_max, num_splits, false).splits;
  if (splits < 1) return 0;
  // enough for either plan: a paged call keeps the split grid
  const size_t split_bytes = mla_workspace((int64_t)B * H, splits);
  const MlaFlat f = plan_mla_flat(B, H, S_max, num_splits, false);
  return f.target > 0 ? std::max(split_bytes, mla_flat_workspace(f, B, H)) : split_bytes;
}

// The split kernel always writes unnormalised partials; the combine divides
// (also for one split) and writes bf16 out and the natural-log lse.
static int run_mla(dattn::MlaArgs& a, int splits, float* lse, uint16_t* out, void* workspace,
                   hipStream_t s, const char* name) {
  const bool flat = a.flat_target > 0;
  const size_t rs = flat ? (size_t)a.flat_slots * a.H : (size_t)a.B * a.H * splits;
  a.num_splits = flat ? 1 : splits;
  a.out = out;
  a.lse = lse;
  a.part_o = (float*)workspace;
  a.part_lse = (float*)((char*)workspace + align256(rs * 512 * sizeof(float)));
  a.part_l = (float*)((char*)a.part_lse + align256(rs * sizeof(float)));
  if (flat) a.flat_table = (int32_t*)((char*)a.part_l + align256(rs * sizeof(float)));
  int rc = launch(name, s, [&] { return dattn::launch_mla(a, s); });
  if (rc) return rc;
  dattn::CombineArgs c{a.part_o, a.part_lse, a.part_l, out, lse, a.B * a.H, splits, 512, 1};
  if (flat) {
    c.items = a.flat_table;
    c.heads = a.H;
    c.splits = mla_flat_full_items(a.B, a.page_table ? (int64_t)a.page_size * a.max_pages : a.S_max,
                                   a.flat_target, a.flat_min, a.flat_max);
  }
  return launch("lse_combine", s, [&] { return dattn::launch_combine(c, s); });
}

int decode_attn_mla(const void* q_absorbed, const void* latent_cache, const int32_t* seq_lens,
                    const int32_t* page_table, void* out, float* lse, int32_t B, int32_t H,
                    int32_t d_latent, int32_t d_rope, int32_t S_max, int32_t page_size,
                    int32_t max_pages, int32_t dtype, float scale, int32_t num_splits,
                    void* workspace, size_t workspace_bytes, void* stream) {
  int rc = validate_mla_common("decode_attn_mla", q_absorbed, latent_cache, out, B, H, d_latent,
                               d_rope, S_max, dtype, scale, num_splits);
  if (rc) return rc;
  if (!seq_lens) return fail(DATTN_EINVAL, "decode_attn_mla: seq_lens is NULL");
  if (page_table) {
    if (!pow2(page_size)) return fail(DATTN_EUNSUPPORTED, "decode_attn_mla: paged cache needs a power-of-two page_size");
    if (max_pages < 1) return fail(DATTN_EINVAL, "decode_attn_mla: max_pages must be >= 1");
    // decode_attn_mla_workspace plans from S_max: both must see one capacity
    if ((int64_t)page_size * max_pages != S_max)
      return fail(DATTN_EINVAL, "decode_attn_mla: paged S_max (%d) must equal page_size * max_pages (%lld)",
                  S_max, (long long)page_size * max_pages);
  }
  const int64_t max_tokens = S_max;
  const MlaPlan plan = plan_mla(B, H, max_tokens, num_splits, false);
  const int splits = plan.splits;
  if (splits < 1) return fail(DATTN_EUNSUPPORTED, "decode_attn_mla: %lld tokens need more than %d splits",
                              (long long)max_tokens, kMlaMaxSplits);
  const MlaFlat flat = plan_mla_flat(B, H, max_tokens, num_splits, page_table != nullptr);
  const size_t need = flat.target > 0 ? mla_flat_workspace(flat, B, H) : mla_workspace((int64_t)B * H, splits);
  if ((rc = check_workspace(workspace, workspace_bytes, need))) return rc;
  if (debug_on()) {
    const void* caches[] = {latent_cache};
    const int64_t pb = (int64_t)page_size * (d_latent + d_rope) * 2;
    if ((rc = debug_check("decode_attn_mla", seq_lens, page_table, B, page_table ? page_size : S_max,
                          page_table ? max_pages : 1, caches, 1, pb, (hipStream_t)stream)))
      return rc;
  }
  dattn::MlaArgs a{};
  a.q = (const uint16_t*)q_absorbed;
  a.latent = (const uint16_t*)latent_cache;
  a.seq_lens = seq_lens;
  a.page_table = page_table;
  a.B = B;
  a.H = H;
  a.heads_per_wg = plan.heads_per_wg;
  a.S_max = S_max;
  a.page_size = page_table ? page_size : S_max;
  a.log2_page = page_table ? ilog2(page_size) : 0;
  a.max_pages = page_table ? max_pages : 1;
  const float sc = scale > 0.f ? scale : 1.0f / std::sqrt(192.0f);
  a.scale_log2 = sc * 1.4426950408889634f;
  if (flat.target > 0) {
    a.flat_target = flat.target;
    a.flat_slots = flat.slots;
    a.flat_min = kMlaDenseMinSplitTokens;
    a.flat_max = dattn::kMlaMaxSplitTokens;
  }
  return run_mla(a, splits, lse, (uint16_t*)out, workspace, (hipStream_t)stream, "mla_split");
}

size_t sparse_mla_attn_workspace(int32_t B, int32_t H, int32_t d_latent, int32_t k, int32_t num_splits) {
  if (B < 1 || H < 64 || H % 64 != 0 || d_latent < 1 || k < 1 || num_splits < 0) return 0;
  const int splits = plan_mla(B, H, k, num_splits, true).splits;
  return splits > 0 ? mla_workspace((int64_t)B * H, splits) : 0;
}

int sparse_mla_attn(const void* q, const void* latent_cache, const int32_t* topk_idx, int32_t k,
                    void* out, float* lse, int32_t B, int32_t H, int32_t d_latent, int32_t d_rope,
                    int32_t S_max, int32_t dtype, float scale, int32_t num_splits, void* workspace,
                    size_t workspace_bytes, void* stream) {
  int rc = validate_mla_common("sparse_mla_attn", q, latent_cache, out, B, H, d_latent, d_rope,
                               S_max, dtype, scale, num_splits);
  if (rc) return rc;
  if (!topk_idx) return fail(DATTN_EINVAL, "sparse_mla_attn: topk_idx is NULL");
  if (k < 1) return fail(DATTN_EINVAL, "sparse_mla_attn: k must be >= 1");
  const MlaPlan plan = plan_mla(B, H, k, num_splits, true);
  const int splits = plan.splits;
  if (splits < 1) return fail(DATTN_EUNSUPPORTED, "sparse_mla_attn: k = %d needs more than %d splits", k,
                              kMlaMaxSplits);
  if ((rc = check_workspace(workspace, workspace_bytes, mla_workspace((int64_t)B * H, splits))))
    return rc;
  dattn::MlaArgs a{};
  a.q = (const uint16_t*)q;
  a.latent = (const uint16_t*)latent_cache;
  a.idx = topk_idx;
  a.k_sel = k;
  a.B = B;
  a.H = H;
  a.heads_per_wg = plan.heads_per_wg;
  a.S_max = S_max;
  a.page_size = S_max;
  a.max_pages = 1;
  const float sc = scale > 0.f ? scale : 1.0f / std::sqrt(192.0f);
  a.scale_log2 = sc * 1.4426950408889634f;
  return run_mla(a, splits, lse, (uint16_t*)out, workspace, (hipStream_t)stream, "sparse_mla_split");
}

// ------------------------------------------------------------------- DSA

size_t dsa_topk_workspace(int32_t B, int32_t S_max, int32_t k) {
  (void)k;
  if (B < 1 || S_max < 1 || S_max > kTopkMaxRow) return 0;
  return dattn::topk_workspace_bytes(B, S_max);
}

int dsa_topk(const float* scores, const int32_t* seq_lens, int32_t k, int32_t* topk_idx, int32_t B,
             int32_t S_max, void* workspace, size_t workspace_bytes, void* stream) {
  if (!scores || !seq_lens || !topk_idx) return fail(DATTN_EINVAL, "dsa_topk: NULL pointer argument");
  if (B < 1 || S_max < 1) return fail(DATTN_EINVAL, "dsa_topk: B and S_max must be >= 1");
  if (B > 65535) return fail(DATTN_EINVAL, "dsa_topk: B must be <= 65535");
  if (S_max > kTopkMaxRow) return fail(DATTN_EINVAL, "dsa_topk: S_max must be <= %d", kTopkMaxRow);
  if (k < 1 || k > kTopkMax) return fail(DATTN_EINVAL, "dsa_topk: k = %d outside [1, %d]", k, kTopkMax);
  int rc = check_workspace(workspace, workspace_bytes, dsa_topk_workspace(B, S_max, k));
  if (rc) return rc;
  dattn::TopkArgs t{scores, seq_lens, topk_idx, B, S_max, k, (uint32_t*)workspace, 0, 0};
  hipStream_t s = (hipStream_t)stream;
  rc = launch("topk_select", s, [&] { return dattn::launch_topk(t, s); });
  return rc ? rc : ok();
}

// [scores fp32 B x S_max, used when scores_out is NULL | top-k workspace]
size_t dsa_indexer_topk_workspace(int32_t B, int32_t S_max, int32_t k) {
  if (B < 1 || S_max < 1 || S_max > kTopkMaxRow) return 0;
  return align256((size_t)B * S_max * sizeof(float)) + dsa_topk_workspace(B, S_max, k);
}

int dsa_indexer_topk(const void* q_i, const float* w, const void* k_i_cache, const int32_t* seq_lens,
                     int32_t k, int32_t* topk_idx, float* scores_out, int32_t B, int32_t Hi,
                     int32_t Di, int32_t S_max, int32_t dtype, void* workspace,
                     size_t workspace_bytes, void* stream) {
  if (!q_i || !w || !k_i_cache || !seq_lens || !topk_idx)
    return fail(DATTN_EINVAL, "dsa_indexer_topk: NULL pointer argument");
  if (!aligned16(q_i) || !aligned16(k_i_cache))
    return fail(DATTN_EINVAL, "dsa_indexer_topk: q_i and k_i_cache must be 16-byte aligned");
  if (B < 1 || S_max < 1) return fail(DATTN_EINVAL, "dsa_indexer_topk: B and S_max must be >= 1");
  if (B > 65535) return fail(DATTN_EINVAL, "dsa_indexer_topk: B must be <= 65535");
  if (k < 1 || k > kTopkMax) return fail(DATTN_EINVAL, "dsa_indexer_topk: k = %d outside [1, %d]", k, kTopkMax);
  if (Di != 128) return fail(DATTN_EUNSUPPORTED, "dsa_indexer_topk: Di = %d; only 128 is built", Di);
  if (Hi != 32 && Hi != 64 && Hi != 96 && Hi != 128)
    return fail(DATTN_EUNSUPPORTED, "dsa_indexer_topk: Hi = %d not in {32,64,96,128}", Hi);
  if (dtype != DATTN_BF16 && dtype != DATTN_FP8_E4M3)
    return fail(DATTN_EUNSUPPORTED, "dsa_indexer_topk: dtype %d; bf16 and fp8 e4m3 are built", dtype);
  if (S_max > kTopkMaxRow)
    return fail(DATTN_EINVAL, "dsa_indexer_topk: S_max must be <= %d", kTopkMaxRow);
  int rc = check_workspace(workspace, workspace_bytes, dsa_indexer_topk_workspace(B, S_max, k));
  if (rc) return rc;
  if (debug_on() && (rc = debug_check("dsa_indexer_topk", seq_lens, nullptr, B, S_max, 1, nullptr, 0, 0,
                                      (hipStream_t)stream)))
    return rc;
  float* scores = scores_out ? scores_out : (float*)workspace;
  uint32_t* topk_ws = (uint32_t*)((char*)workspace + align256((size_t)B * S_max * sizeof(float)));
  hipStream_t s = (hipStream_t)stream;
  dattn::IndexerArgs ia{q_i,   w, k_i_cache, seq_lens, scores, B, Hi, S_max, 0, dtype == DATTN_FP8_E4M3,
                        topk_ws, dattn::topk_row_words_of(S_max)};
  rc = launch("indexer_scores", s, [&] { return dattn::launch_indexer(ia, s); });
  if (rc) return rc;
  dattn::TopkArgs t{scores, seq_lens, topk_idx, B, S_max, k, topk_ws, 0, 0};
  t.hist0_done = ia.hist0 != nullptr;  // the indexer wrote the first level
  rc = launch("topk_select", s, [&] { return dattn::launch_topk(t, s); });
  return rc ? rc : ok();
}

}  // extern "C"

// ------------------------------------------------------------------- Quest

namespace {

// Summary slots per sequence: the full 16-token blocks the cache can hold.
int64_t quest_blocks(int32_t page_size, int32_t max_pages, bool paged) {
  return (int64_t)page_size * (paged ? max_pages : 1) / 16;
}

int validate_quest_cache(const char* fn, const void* k, const void* kminmax, const int32_t* seq_lens,
                         const int32_t* page_table, int32_t B, int32_t Hkv, int32_t D,
                         int32_t page_size, int32_t max_pages, int32_t dtype) {
  if (!k || !kminmax || !seq_lens) return fail(DATTN_EINVAL, "%s: NULL pointer argument", fn);
  if (!aligned16(k) || !aligned16(kminmax)) return fail(DATTN_EINVAL, "%s: k_cache and kminmax must be 16-byte aligned", fn);
  if (B < 1 || Hkv < 1) return fail(DATTN_EINVAL, "%s: B and Hkv must be >= 1", fn);
  if (B > 65535 || Hkv > 65535) return fail(DATTN_EINVAL, "%s: B and Hkv must be <= 65535", fn);
  if (D != 64 && D != 128) return fail(DATTN_EUNSUPPORTED, "%s: head dim %d not in {64,128}", fn, D);
  if (dtype != DATTN_F32 && dtype != DATTN_BF16) return fail(DATTN_EUNSUPPORTED, "%s: dtype %d", fn, dtype);
  if (page_size < 1) return fail(DATTN_EINVAL, "%s: page_size must be >= 1", fn);
  if (page_table) {
    if (!pow2(page_size) || page_size < 16)
      return fail(DATTN_EUNSUPPORTED, "%s: paged cache needs a power-of-two page_size >= 16, got %d", fn, page_size);
    if (max_pages < 1) return fail(DATTN_EINVAL, "%s: max_pages must be >= 1", fn);
  }
  if (quest_blocks(page_size, max_pages, page_table != nullptr) >= ((int64_t)1 << 31))
    return fail(DATTN_EINVAL, "%s: too many 16-token blocks per sequence", fn);
  return DATTN_OK;
}

dattn::QuestArgs quest_args(const void* q, const void* k, const void* kminmax, const int32_t* seq_lens,
                            const int32_t* page_table, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                            int32_t page_size, int32_t max_pages, int32_t dtype) {
  dattn::QuestArgs a{};
  a.q = q;
  a.k = k;
  a.kminmax = const_cast<void*>(kminmax);
  a.seq_lens = seq_lens;
  a.page_table = page_table;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = D;
  a.G = Hq / Hkv;
  a.page_size = page_size;
  a.log2_page = page_table ? ilog2(page_size) : 0;
  a.max_pages = page_table ? max_pages : 1;
  a.max_blocks = (int32_t)quest_blocks(page_size, max_pages, page_table != nullptr);
  a.bf16 = dtype == DATTN_BF16;
  return a;
}

// The attention reads each chosen block once per group of query heads (the
// union of their choices) when the group has more than one head and the
// per-head bitmaps fit the union kernel; else one query head per workgroup.
struct QuestPlan {
  bool uni;
  int splits;
  int32_t cap;  // union entries per (sequence, KV head)
  size_t upper, n_full, sel, topk, ulist, ucount, parts, total;  // byte offsets of the workspace parts
};

QuestPlan plan_quest(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int64_t max_blocks, int32_t budget,
                     bool bf16, int32_t num_splits, bool own_sel) {
  QuestPlan p{};
  const int G = Hq / Hkv;
  const int64_t rows = (int64_t)B * Hq;
  const int64_t kept = budget < max_blocks ? budget : max_blocks;
  p.uni = G > 1 && max_blocks > 0 && max_blocks <= dattn::kQuestUnionMaxBlocks;
  p.cap = p.uni ? (int32_t)std::min<int64_t>((int64_t)G * budget, max_blocks) : 0;
  const int64_t units = p.uni ? (int64_t)B * Hkv : rows;
  const int64_t max_tokens = 16 * ((p.uni ? p.cap : kept) + 1);  // the chosen blocks and the partial one
  const int64_t slots =
      num_splits > 0 ? 0
                     : (int64_t)std::min(std::max(dattn::gqa_listed_blocks_per_cu(bf16, D, G, p.uni), 3),
                                         kMaxSplitWgPerCu) *
                           dattn::device_cu_count();
  p.splits = plan_gqa_splits((int32_t)units, 1, max_tokens, num_splits, slots);
  const int64_t nb = max_blocks > 0 ? max_blocks : 1;
  p.upper = 0;
  p.n_full = p.upper + align256((size_t)rows * nb * sizeof(float));
  p.sel = p.n_full + align256((size_t)rows * sizeof(int32_t));
  p.topk = p.sel + (own_sel ? align256((size_t)rows * budget * sizeof(int32_t)) : 0);
  p.ulist = p.topk + dattn::topk_workspace_bytes((int)rows, (int)nb);
  p.ucount = p.ulist + (p.uni ? align256((size_t)B * Hkv * p.cap * sizeof(int32_t)) : 0);
  p.parts = p.ucount + (p.uni ? align256((size_t)B * Hkv * sizeof(int32_t)) : 0);
  p.total = p.parts + split_workspace(rows, p.splits, D);
  return p;
}

}  // namespace

extern "C" {

int quest_page_minmax(const void* k_cache, const int32_t* seq_lens, const int32_t* page_table,
                      void* kminmax, int32_t first_block, int32_t B, int32_t Hkv, int32_t D,
                      int32_t page_size, int32_t max_pages, int32_t dtype, void* stream) {
  int rc = validate_quest_cache("quest_page_minmax", k_cache, kminmax, seq_lens, page_table, B, Hkv, D,
                                page_size, max_pages, dtype);
  if (rc) return rc;
  if (first_block < 0) return fail(DATTN_EINVAL, "quest_page_minmax: first_block must be >= 0");
  dattn::QuestArgs a = quest_args(nullptr, k_cache, kminmax, seq_lens, page_table, B, Hkv, Hkv, D,
                                  page_size, max_pages, dtype);
  a.first_block = first_block;
  hipStream_t s = (hipStream_t)stream;
  if ((rc = launch("quest_minmax", s, [&] { return dattn::launch_quest_minmax(a, s); }))) return rc;
  return ok();
}

size_t decode_attn_quest_workspace(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t page_size,
                                   int32_t max_pages, int32_t budget, int32_t dtype, int32_t num_splits) {
  if (B < 1 || Hq < 1 || Hkv < 1 || D < 1 || page_size < 1 || max_pages < 1 || budget < 1 ||
      num_splits < 0)
    return 0;
  if (Hq % Hkv != 0) return 0;
  const QuestPlan p = plan_quest(B, Hq, Hkv, D, quest_blocks(page_size, max_pages, true), budget,
                                 dtype == DATTN_BF16, num_splits, true);
  return p.total;
}

int decode_attn_quest(const void* q, const void* k_cache, const void* v_cache, const void* kminmax,
                      const int32_t* seq_lens, const int32_t* page_table, int32_t budget, void* out,
                      float* lse, int32_t* selected, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                      int32_t page_size, int32_t max_pages, int32_t dtype, float scale, int32_t num_splits,
                      void* workspace, size_t workspace_bytes, void* stream) {
  int rc = validate_gqa(q, k_cache, v_cache, seq_lens, page_table, 0, out, B, Hq, Hkv, D, page_size,
                        max_pages, dtype, scale, num_splits);
  if (rc) return rc;
  if ((rc = validate_quest_cache("decode_attn_quest", k_cache, kminmax, seq_lens, page_table, B, Hkv, D,
                                 page_size, max_pages, dtype)))
    return rc;
  if (budget < 1 || budget > kTopkMax)
    return fail(DATTN_EINVAL, "decode_attn_quest: budget = %d pages outside [1, %d]", budget, kTopkMax);
  if ((int64_t)B * Hq > 65535) return fail(DATTN_EINVAL, "decode_attn_quest: B * Hq must be <= 65535");
  const bool paged = page_table != nullptr;
  dattn::QuestArgs qa = quest_args(q, k_cache, kminmax, seq_lens, page_table, B, Hq, Hkv, D, page_size,
                                   max_pages, dtype);
  const QuestPlan p = plan_quest(B, Hq, Hkv, D, qa.max_blocks, budget, dtype == DATTN_BF16, num_splits,
                                 selected == nullptr);
  if ((rc = check_workspace(workspace, workspace_bytes, p.total))) return rc;
  if (debug_on()) {
    const void* caches[] = {k_cache, v_cache};
    const int64_t pb = (int64_t)Hkv * page_size * D * (dtype == DATTN_BF16 ? 2 : 4);
    if ((rc = debug_check("decode_attn_quest", seq_lens, page_table, B, page_size, paged ? max_pages : 1,
                          caches, 2, pb, (hipStream_t)stream)))
      return rc;
  }
  char* ws = (char*)workspace;
  hipStream_t s = (hipStream_t)stream;
  int32_t* sel = selected ? selected : (int32_t*)(ws + p.sel);
  qa.upper = (float*)(ws + p.upper);
  qa.n_full = (int32_t*)(ws + p.n_full);
  if (qa.max_blocks > 0) {
    if ((rc = launch("quest_bounds", s, [&] { return dattn::launch_quest_bounds(qa, s); }))) return rc;
    dattn::TopkArgs t{qa.upper, qa.n_full, sel, B * Hq, qa.max_blocks, budget, (uint32_t*)(ws + p.topk), 0, 0};
    if ((rc = launch("topk_select", s, [&] { return dattn::launch_topk(t, s); }))) return rc;
  }
  if (p.uni) {
    dattn::QuestUnionArgs u{sel, seq_lens, (int32_t*)(ws + p.ulist), (int32_t*)(ws + p.ucount), B, Hq, Hkv,
                            Hq / Hkv, budget, p.cap, qa.max_blocks};
    if ((rc = launch("quest_union", s, [&] { return dattn::launch_quest_union(u, s); }))) return rc;
  }

  dattn::GqaArgs a{};
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.seq_lens = seq_lens;
  a.page_table = page_table;
  a.out = out;
  a.lse = lse;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = D;
  a.G = Hq / Hkv;
  a.page_size = page_size;
  a.log2_page = paged ? ilog2(page_size) : 0;
  a.max_pages = paged ? max_pages : 1;
  a.num_splits = p.splits;
  a.bf16 = dtype == DATTN_BF16;
  const float sc = scale > 0.f ? scale : 1.0f / std::sqrt((float)D);
  a.scale_log2 = sc * 1.4426950408889634f;
  if (p.uni) {
    a.block_list = (const int32_t*)(ws + p.ulist);
    a.list_len = p.cap;
    a.list_count = (const int32_t*)(ws + p.ucount);
  } else {
    a.block_list = sel;
    a.list_len = qa.max_blocks > 0 ? budget : 0;
  }
  if (p.splits > 1) {
    a.part_o = (float*)(ws + p.parts);
    a.part_lse = (float*)(ws + p.parts + align256((size_t)B * Hq * p.splits * D * sizeof(float)));
  }
  if ((rc = launch("gqa_split", s, [&] { return dattn::launch_gqa(a, s); }))) return rc;
  if (p.splits > 1) {
    dattn::CombineArgs c{a.part_o, a.part_lse, nullptr, out, lse, B * Hq, p.splits, D, a.bf16};
    if ((rc = launch("lse_combine", s, [&] { return dattn::launch_combine(c, s); }))) return rc;
  }
  return ok();
}

}  // extern "C"

extern "C" {

// ------------------------------------------------------------- cache append
static int append_common(const char* fn, const void* ptrs[], int n_ptrs, const int32_t* positions,
                         int32_t B, int32_t heads, int64_t row_bytes, bool paged, int32_t page_size,
                         int32_t max_pages, int32_t dtype) {
  for (int i = 0; i < n_ptrs; ++i) {
    if (!ptrs[i]) return fail(DATTN_EINVAL, "%s: NULL pointer argument", fn);
    if ((uintptr_t)ptrs[i] % 16 != 0) return fail(DATTN_EINVAL, "%s: buffers must be 16-byte aligned", fn);
  }
  if (!positions) return fail(DATTN_EINVAL, "%s: NULL pointer argument", fn);
  if (B < 1 || B > 65535) return fail(DATTN_EINVAL, "%s: B must be in [1, 65535]", fn);
  if (heads < 1) return fail(DATTN_EINVAL, "%s: head count must be >= 1", fn);
  if (dtype != DATTN_F32 && dtype != DATTN_BF16) return fail(DATTN_EUNSUPPORTED, "%s: dtype %d", fn, dtype);
  if (row_bytes < 16 || row_bytes % 16 != 0 || row_bytes > (1 << 20))
    return fail(DATTN_EUNSUPPORTED, "%s: a row of %lld bytes is not a multiple of 16", fn, (long long)row_bytes);
  if (page_size < 1) return fail(DATTN_EINVAL, "%s: page_size must be >= 1", fn);
  if (paged) {
    if (!pow2(page_size)) return fail(DATTN_EUNSUPPORTED, "%s: paged cache needs a power-of-two page_size", fn);
    if (max_pages < 1) return fail(DATTN_EINVAL, "%s: max_pages must be >= 1", fn);
  }
  return DATTN_OK;
}

int kv_append_gqa(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                  const int32_t* positions, int32_t* page_table, int32_t B, int32_t Hkv, int32_t D,
                  int32_t page_size, int32_t max_pages, int32_t ring_pages, int32_t fixed_pages,
                  int32_t dtype, void* stream) {
  const void* ptrs[] = {k_new, v_new, k_cache, v_cache};
  const int64_t esz = dtype == DATTN_BF16 ? 2 : 4;
  int rc = append_common("kv_append_gqa", ptrs, 4, positions, B, Hkv, (int64_t)D * esz,
                         page_table != nullptr, page_size, max_pages, dtype);
  if (rc) return rc;
  if (D < 1) return fail(DATTN_EINVAL, "kv_append_gqa: D must be >= 1");
  if (ring_pages < 0 || fixed_pages < 0)
    return fail(DATTN_EINVAL, "kv_append_gqa: ring_pages and fixed_pages must be >= 0");
  if (ring_pages > 0 && !page_table)
    return fail(DATTN_EINVAL, "kv_append_gqa: a rolling buffer needs a page table");
  dattn::KvAppendArgs a{k_new, v_new, k_cache, v_cache, positions, page_table, B, Hkv,
                        (int32_t)(D * esz), page_size, page_table ? ilog2(page_size) : 0,
                        page_table ? max_pages : 1, ring_pages, fixed_pages};
  hipStream_t s = (hipStream_t)stream;
  rc = launch("kv_append", s, [&] { return dattn::launch_kv_append(a, s); });
  return rc ? rc : ok();
}

int kv_append_rows(const void* rows_new, void* cache, const int32_t* positions,
                   const int32_t* page_table, int32_t B, int32_t row_elems, int32_t page_size,
                   int32_t max_pages, int32_t dtype, void* stream) {
  const void* ptrs[] = {rows_new, cache};
  const int64_t esz = dtype == DATTN_BF16 ? 2 : 4;
  int rc = append_common("kv_append_rows", ptrs, 2, positions, B, 1, (int64_t)row_elems * esz,
                         page_table != nullptr, page_size, max_pages, dtype);
  if (rc) return rc;
  dattn::KvAppendArgs a{rows_new, nullptr, cache, nullptr, positions, (int32_t*)page_table, B, 1,
                        (int32_t)(row_elems * esz), page_size, page_table ? ilog2(page_size) : 0,
                        page_table ? max_pages : 1, 0, 0};
  hipStream_t s = (hipStream_t)stream;
  rc = launch("kv_append", s, [&] { return dattn::launch_kv_append(a, s); });
  return rc ? rc : ok();
}

}  // extern "C"
