// pakv.hip - host side of libpakv: argument validation, pool descriptor,
// split/workspace sizing and kernel launches on the caller's stream.
// The C ABI and the memory layout are documented in include/pakv.h.
#include "pakv.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <climits>
#include <cmath>
#include <cstdint>
#include <new>
#include <queue>
#include <vector>

#include "pakv_kernels.h"
#include "pakv_prefill.h"

struct pa_pool {
  void* k;
  void* v;
  int32_t num_pages;
  int32_t num_kv_heads;
  int32_t head_dim;
};

// Scratch of the allocation-free decode (pa_decode_static): the split
// partials (accumulators, then max and sum) of sequences with more splits
// than one workgroup merges itself. Each device holds its own copy for the
// life of the process. In host code this name stands for no device address:
// the kernels get the address hipGetSymbolAddress gives on each device.
constexpr size_t kStaticScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

constexpr int kMaxGroup = 16;   // query heads per KV head: the 16 MFMA columns
constexpr int kProfileKinds = 5;  // decode, merge, append, chunk write, prefill
constexpr int64_t kPlanMaxSeqs = 1 << 20;   // plan items pack b in 20 bits
// MI355X geometry used by the launch plan's ordering (not by correctness)
constexpr int kDeviceCUs = 256;
constexpr int kCUsPerXCD = 32;
constexpr int64_t kPlanMaxSplits = 1 << 11; // and the split in the 11 above them

// The kernels work with scores in log2 units: scale * log2(e) must be a
// finite FP32 value.
float scale_log2_of(float scale) { return static_cast<float>(static_cast<double>(scale) * 1.4426950408889634); }
bool scale_ok(float scale) { return std::isfinite(scale) && std::isfinite(scale_log2_of(scale)); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int split_pages(int d) {
  return d == 64 ? pakv::DecodeGeom<64>::SPLIT_PAGES : pakv::DecodeGeom<128>::SPLIT_PAGES;
}
int decode_waves(int d) { return d == 64 ? pakv::DecodeGeom<64>::W : pakv::DecodeGeom<128>::W; }

// prefill workgroups (4 waves) one CU holds at once
int prefill_wgs_per_cu(int d) {
  return d == 64 ? pakv::prefill_occupancy<64>() : pakv::prefill_occupancy<128>();
}

// decode workgroups one CU holds at once (waves per SIMD x 4 SIMDs / waves per workgroup)
int decode_wgs_per_cu(int d) { return std::max(1, pakv::occupancy(d) * 4 / decode_waves(d)); }

// The device address of the current device's scratch copy, looked up with
// that device current on its first use and kept per device.
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

pa_status static_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PA_ERR_LAUNCH;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PA_ERR_LAUNCH;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return PA_OK;
}

// Workgroups per KV head that the device holds at once: the bins of a plan.
int64_t decode_slots(const pa_pool* pool) {
  return std::max<int64_t>(1, static_cast<int64_t>(kDeviceCUs) * decode_wgs_per_cu(pool->head_dim) /
                                  pool->num_kv_heads);
}

int64_t splits_for(int d, int32_t max_pages_per_seq) {
  const int64_t sp = split_pages(d);
  return (static_cast<int64_t>(max_pages_per_seq) + sp - 1) / sp;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workspace: partial accumulators [B][Hq][S][D] then (m, l) pairs [B][Hq][S][2],
// needed only when a sequence can have more splits than a work item holds.
void workspace_parts(int d, int32_t num_seqs, int32_t num_q_heads, int group, int32_t max_pages_per_seq,
                     size_t* acc_bytes, size_t* total) {
  const int64_t s = splits_for(d, max_pages_per_seq);
  if (s <= pakv::units_cap(group)) {
    *acc_bytes = 0;
    *total = 0;
    return;
  }
  const size_t items = static_cast<size_t>(num_seqs) * num_q_heads * s;
  *acc_bytes = align_up(items * d * sizeof(float), 256);
  *total = *acc_bytes + align_up(items * 2 * sizeof(float), 256);
}

// ---- optional event timing of each launch (measurement only)
struct ProfileRec {
  hipEvent_t start, stop;
  int kind;
};
bool g_profiling = false;
std::vector<ProfileRec> g_records;
std::vector<hipEvent_t> g_free_events;

hipEvent_t take_event() {
  if (!g_free_events.empty()) {
    hipEvent_t e = g_free_events.back();
    g_free_events.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

struct LaunchTimer {
  ProfileRec rec{nullptr, nullptr, 0};
  hipStream_t stream;
  LaunchTimer(int kind, hipStream_t s) : stream(s) {
    if (!g_profiling) return;
    rec.kind = kind;
    rec.start = take_event();
    rec.stop = take_event();
    if (!rec.start || !rec.stop) {   // keep whichever event was made for later
      if (rec.start) g_free_events.push_back(rec.start);
      if (rec.stop) g_free_events.push_back(rec.stop);
      rec.start = rec.stop = nullptr;
      return;
    }
    (void)hipEventRecord(rec.start, stream);
  }
  ~LaunchTimer() {
    if (!g_profiling || !rec.start) return;
    (void)hipEventRecord(rec.stop, stream);
    try {
      g_records.push_back(rec);
    } catch (...) {   // out of host memory: this launch goes untimed
      (void)hipEventDestroy(rec.start);
      (void)hipEventDestroy(rec.stop);
    }
  }
};

template <int D, int NW>
pa_status launch_decode_with(const pakv::DecodeArgs& args, const pakv::InlinePlan<NW>& ip, int64_t items,
                             int64_t bins, hipStream_t stream) {
  (void)hipGetLastError();
  if (items == 0) return PA_OK;
  if (items > INT_MAX) return PA_ERR_INVALID;
  {
    LaunchTimer t(0, stream);
    // x: KV head, (y, z): bin (y below 65536)
    const unsigned gy = static_cast<unsigned>(std::min<int64_t>(bins, 65535));
    const unsigned gz = static_cast<unsigned>((bins + 65534) / 65535);
    pakv::DecodeArgs a = args;
    a.num_items = static_cast<int32_t>(items);
    a.num_bins = static_cast<int32_t>(bins);
    // a chain can only reach items past the bins' first ones
    if (items > bins)
      hipLaunchKernelGGL((pakv::decode_kernel<D, NW, true>), dim3(static_cast<unsigned>(args.num_kv_heads), gy, gz),
                         dim3(64 * pakv::DecodeGeom<D>::W), 0, stream, a, ip);
    else
      hipLaunchKernelGGL((pakv::decode_kernel<D, NW, false>), dim3(static_cast<unsigned>(args.num_kv_heads), gy, gz),
                         dim3(64 * pakv::DecodeGeom<D>::W), 0, stream, a, ip);
  }
  if (hipGetLastError() != hipSuccess) return PA_ERR_LAUNCH;
  if (args.s_max > args.ucap) {
    const int64_t heads = static_cast<int64_t>(args.num_seqs) * args.num_q_heads;
    const int64_t mblocks = (heads + 3) / 4;
    if (mblocks > INT_MAX) return PA_ERR_INVALID;
    {
      LaunchTimer t(1, stream);
      hipLaunchKernelGGL((pakv::merge_splits_kernel<D>), dim3(static_cast<unsigned>(mblocks)), dim3(256),
                         0, stream, args);
    }
    if (hipGetLastError() != hipSuccess) return PA_ERR_LAUNCH;
  }
  return PA_OK;
}

// plan_host: a host plan of plan_ints words to carry in the launch's
// arguments (NULL: the device plan in args, or none)
template <int D>
pa_status launch_decode(const pakv::DecodeArgs& args, const int32_t* plan_host, int32_t plan_ints, int64_t items,
                        int64_t bins, hipStream_t stream) {
  if (plan_host && plan_ints <= pakv::kInlineSmall) {
    pakv::InlinePlan<pakv::kInlineSmall> ip;
    std::copy(plan_host, plan_host + plan_ints, ip.w);
    std::fill(ip.w + plan_ints, ip.w + pakv::kInlineSmall, 0);
    return launch_decode_with<D>(args, ip, items, bins, stream);
  }
  if (plan_host) {
    pakv::InlinePlan<pakv::kInlineLarge> ip;
    std::copy(plan_host, plan_host + plan_ints, ip.w);
    std::fill(ip.w + plan_ints, ip.w + pakv::kInlineLarge, 0);
    return launch_decode_with<D>(args, ip, items, bins, stream);
  }
  pakv::InlinePlan<pakv::kItemInts> none{};
  return launch_decode_with<D>(args, none, items, bins, stream);
}

}  // namespace

extern "C" {

const char* pa_status_str(pa_status s) {
  switch (s) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "a required pointer is NULL";
    case PA_ERR_INVALID: return "a count or size is out of range";
    case PA_ERR_UNSUPPORTED: return "unsupported page size, head_dim or query-head group size";
    case PA_ERR_ALIGN: return "a device pointer is not aligned as documented";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_LAUNCH: return "the HIP runtime failed to queue a kernel";
    case PA_ERR_CAPACITY: return "the request needs more pages than the whole pool: rejected";
    case PA_ERR_STATE: return "the request is not in a state that allows this call";
  }
  return "unknown status";
}

pa_status pa_pool_create(pa_pool** out, void* k_pages, void* v_pages, int32_t num_pages,
                         int32_t page_size, int32_t num_kv_heads, int32_t head_dim) {
  if (!out) return PA_ERR_NULL;
  *out = nullptr;
  if (!k_pages || !v_pages) return PA_ERR_NULL;
  if (num_pages < 1 || num_kv_heads < 1 || page_size < 1 || head_dim < 1) return PA_ERR_INVALID;
  if (page_size != pakv::kPage) return PA_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (!aligned16(k_pages) || !aligned16(v_pages)) return PA_ERR_ALIGN;
  pa_pool* p = new (std::nothrow) pa_pool;
  if (!p) return PA_ERR_INVALID;
  p->k = k_pages;
  p->v = v_pages;
  p->num_pages = num_pages;
  p->num_kv_heads = num_kv_heads;
  p->head_dim = head_dim;
  *out = p;
  return PA_OK;
}

void pa_pool_destroy(pa_pool* pool) { delete pool; }

int32_t pa_split_tokens(int32_t head_dim) {
  if (head_dim != 64 && head_dim != 128) return 0;
  return split_pages(head_dim) * pakv::kPage;
}

size_t pa_decode_workspace_bytes(const pa_pool* pool, int32_t num_seqs, int32_t num_q_heads,
                                 int32_t max_pages_per_seq) {
  if (!pool || num_seqs <= 0 || num_q_heads <= 0 || max_pages_per_seq <= 0) return 0;
  if (num_q_heads % pool->num_kv_heads != 0) return 0;
  size_t acc = 0, total = 0;
  workspace_parts(pool->head_dim, num_seqs, num_q_heads, num_q_heads / pool->num_kv_heads, max_pages_per_seq,
                  &acc, &total);
  return total;
}

pa_status pa_kv_append(const pa_pool* pool, const void* k_new, const void* v_new, int32_t num_seqs,
                       const int32_t* block_tables, int32_t max_pages_per_seq,
                       const int32_t* positions, void* stream) {
  if (!pool) return PA_ERR_NULL;
  if (num_seqs < 0 || max_pages_per_seq < 1) return PA_ERR_INVALID;
  if (static_cast<int64_t>(max_pages_per_seq) * pakv::kPage > INT_MAX) return PA_ERR_INVALID;
  if (num_seqs == 0) return PA_OK;
  if (!k_new || !v_new || !block_tables || !positions) return PA_ERR_NULL;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned4(block_tables) || !aligned4(positions))
    return PA_ERR_ALIGN;
  pakv::AppendArgs a;
  a.kpool = static_cast<uint16_t*>(pool->k);
  a.vpool = static_cast<uint16_t*>(pool->v);
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.block_tables = block_tables;
  a.positions = positions;
  a.num_pages = pool->num_pages;
  a.num_seqs = num_seqs;
  a.num_kv_heads = pool->num_kv_heads;
  a.stride = max_pages_per_seq;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const unsigned blocks = static_cast<unsigned>(num_seqs);
  (void)hipGetLastError();
  {
    LaunchTimer t(2, s);
    if (pool->head_dim == 64)
      hipLaunchKernelGGL((pakv::kv_append_kernel<64>), dim3(blocks), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((pakv::kv_append_kernel<128>), dim3(blocks), dim3(256), 0, s, a);
  }
  if (hipGetLastError() != hipSuccess) return PA_ERR_LAUNCH;
  return PA_OK;
}

static pa_status decode_impl(const pa_pool* pool, const void* q, int32_t num_seqs, int32_t num_q_heads,
                             const int32_t* block_tables, int32_t max_pages_per_seq,
                             const int32_t* context_lens, float scale, float* out, void* workspace,
                             size_t workspace_bytes, const int32_t* plan, const int32_t* plan_host,
                             int32_t plan_ints, void* stream) {
  if (!pool) return PA_ERR_NULL;
  if (num_seqs < 0 || num_q_heads < 1 || max_pages_per_seq < 1) return PA_ERR_INVALID;
  if (static_cast<int64_t>(max_pages_per_seq) * pakv::kPage > INT_MAX) return PA_ERR_INVALID;
  if (!scale_ok(scale)) return PA_ERR_INVALID;
  if (num_q_heads % pool->num_kv_heads != 0) return PA_ERR_INVALID;
  const int group = num_q_heads / pool->num_kv_heads;
  if (group > kMaxGroup) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PA_OK;
  if (!q || !block_tables || !context_lens || !out) return PA_ERR_NULL;
  if (!aligned16(q) || !aligned4(block_tables) || !aligned4(context_lens) || !aligned16(out))
    return PA_ERR_ALIGN;
  const int d = pool->head_dim;
  const int64_t s_max = splits_for(d, max_pages_per_seq);
  if (num_seqs > kPlanMaxSeqs || s_max > kPlanMaxSplits) {
    if (plan || plan_host) return PA_ERR_INVALID;
  }
  if (plan_ints < 0 || plan_ints % pakv::kItemInts != 0) return PA_ERR_INVALID;
  if (plan_ints > static_cast<int64_t>(num_seqs) * s_max * pakv::kItemInts) return PA_ERR_INVALID;
  if (plan_host && plan_ints > pakv::kInlineLarge) return PA_ERR_INVALID;
  if (plan_ints > 0 && !plan && !plan_host) return PA_ERR_NULL;
  if (plan && !aligned4(plan)) return PA_ERR_ALIGN;
  size_t acc_bytes = 0, need = 0;
  workspace_parts(d, num_seqs, num_q_heads, group, max_pages_per_seq, &acc_bytes, &need);
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return PA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return PA_ERR_ALIGN;
  }
  pakv::DecodeArgs a;
  a.kpool = static_cast<const uint16_t*>(pool->k);
  a.vpool = static_cast<const uint16_t*>(pool->v);
  a.q = static_cast<const uint16_t*>(q);
  a.block_tables = block_tables;
  a.ctx = context_lens;
  a.out = out;
  a.ws_acc = need ? static_cast<float*>(workspace) : nullptr;
  a.ws_ml = need ? reinterpret_cast<float*>(static_cast<char*>(workspace) + acc_bytes) : nullptr;
  a.num_pages = pool->num_pages;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = pool->num_kv_heads;
  a.group = group;
  a.stride = max_pages_per_seq;
  a.s_max = static_cast<int32_t>(s_max);
  a.ucap = pakv::units_cap(group);
  a.scale_log2 = scale_log2_of(scale);
  a.plan = plan_host ? nullptr : plan;
  // work items: the plan's (the first min(slots, items) of them head the
  // bins' chains), or per sequence its splits in groups of ucap, one item
  // per workgroup
  const bool planned = plan || plan_host;
  const int64_t items = planned ? plan_ints / pakv::kItemInts
                                : static_cast<int64_t>(num_seqs) * ((s_max + a.ucap - 1) / a.ucap);
  const int64_t bins = planned ? std::min(items, decode_slots(pool)) : items;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (d == 64) return launch_decode<64>(a, plan_host, plan_ints, items, bins, s);
  return launch_decode<128>(a, plan_host, plan_ints, items, bins, s);
}

pa_status pa_decode(const pa_pool* pool, const void* q, int32_t num_seqs, int32_t num_q_heads,
                    const int32_t* block_tables, int32_t max_pages_per_seq,
                    const int32_t* context_lens, float scale, float* out, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return decode_impl(pool, q, num_seqs, num_q_heads, block_tables, max_pages_per_seq, context_lens, scale, out,
                     workspace, workspace_bytes, nullptr, nullptr, 0, stream);
}

int64_t pa_decode_plan_capacity(const pa_pool* pool, int32_t num_seqs, int32_t max_pages_per_seq) {
  if (!pool || num_seqs < 0 || max_pages_per_seq < 1) return -1;
  const int64_t s_max = splits_for(pool->head_dim, max_pages_per_seq);
  if (num_seqs > kPlanMaxSeqs || s_max > kPlanMaxSplits) return -1;
  return static_cast<int64_t>(num_seqs) * s_max * pakv::kItemInts;
}

static pa_status decode_plan_impl(const pa_pool* pool, const int32_t* context_lens_host, int32_t num_seqs,
                                  int group, int32_t max_pages_per_seq, int32_t* plan, int64_t capacity,
                                  int32_t* num_ints);

pa_status pa_decode_plan(const pa_pool* pool, const int32_t* context_lens_host, int32_t num_seqs,
                         int32_t num_q_heads, int32_t max_pages_per_seq, int32_t* plan, int64_t capacity,
                         int32_t* num_ints) {
  if (!pool || !num_ints) return PA_ERR_NULL;
  *num_ints = 0;
  const int64_t cap_needed = pa_decode_plan_capacity(pool, num_seqs, max_pages_per_seq);
  if (cap_needed < 0) return PA_ERR_INVALID;
  if (num_q_heads < 1 || num_q_heads % pool->num_kv_heads != 0) return PA_ERR_INVALID;
  const int group = num_q_heads / pool->num_kv_heads;
  if (group > kMaxGroup) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PA_OK;
  if (!context_lens_host || !plan) return PA_ERR_NULL;
  try {
    return decode_plan_impl(pool, context_lens_host, num_seqs, group, max_pages_per_seq, plan, capacity,
                            num_ints);
  } catch (...) {   // out of host memory; nothing escapes the C ABI
    *num_ints = 0;
    return PA_ERR_INVALID;
  }
}

// The plan packs units (splits of one sequence) into work items of at most
// ucap units, and items into bins, one workgroup per bin and KV head that
// runs its bin's items in turn:
//  - a sequence of at most ucap splits is one indivisible group (its splits
//    are merged inside the workgroup); a longer one gives one group per
//    split (merged by the merge kernel);
//  - a group costs its pairs plus kUnitCost per unit (an item's fixed work,
//    the start of its stream and its merge, shared by its units; 2 measured
//    a little faster than 0, 5, 10 or 20 on the 16-layer step); groups go,
//    costliest first, each to the bin of least cost so far, over as many
//    bins as the device holds workgroups at once (or one per group, if there
//    are fewer groups), so that the bins end together;
//  - in each bin, its groups in that order go to the first of its items with
//    room for them (a new item when none has);
//  - item b (b < bins) is bin b's first item; each item names the bin's next
//    one, listed after all the first items.
// A unit's rotation is the number of pairs before it in its item, mod W:
// the workgroup's waves then deal all of the item's pairs round-robin.
constexpr int64_t kUnitCost = 2;

static pa_status decode_plan_impl(const pa_pool* pool, const int32_t* context_lens_host, int32_t num_seqs,
                                  int group, int32_t max_pages_per_seq, int32_t* plan, int64_t capacity,
                                  int32_t* num_ints) {
  const int d = pool->head_dim;
  const int sp = split_pages(d);
  const int W = decode_waves(d);
  const int ucap = pakv::units_cap(group);
  const int64_t max_tok = static_cast<int64_t>(max_pages_per_seq) * pakv::kPage;
  struct Group {
    int64_t pairs, cost;
    int32_t b, s0, units;
  };
  auto split_pairs = [&](int64_t pages, int64_t s) {
    return (std::min<int64_t>(pages - s * sp, sp) + 1) / 2;
  };
  std::vector<Group> groups;
  groups.reserve(static_cast<size_t>(num_seqs));
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int64_t n = std::min<int64_t>(std::max(context_lens_host[b], 0), max_tok);
    const int64_t pages = (n + pakv::kPage - 1) / pakv::kPage;
    const int64_t ns = (pages + sp - 1) / sp;
    if (ns <= 1) {   // an empty context keeps one unit: it writes the zero output
      const int64_t p = ns ? split_pairs(pages, 0) : 0;
      groups.push_back({p, p + kUnitCost, b, 0, 1});
    } else if (ns <= ucap) {
      int64_t p = 0;
      for (int64_t s = 0; s < ns; ++s) p += split_pairs(pages, s);
      groups.push_back({p, p + kUnitCost * ns, b, 0, static_cast<int32_t>(ns)});
    } else {
      for (int64_t s = 0; s < ns; ++s) {
        const int64_t p = split_pairs(pages, s);
        groups.push_back({p, p + kUnitCost, b, static_cast<int32_t>(s), 1});
      }
    }
  }
  std::stable_sort(groups.begin(), groups.end(), [](const Group& x, const Group& y) { return x.cost > y.cost; });
  const int64_t nb = std::min<int64_t>(static_cast<int64_t>(groups.size()), decode_slots(pool));
  // groups to bins: least cost first, ties to the lower bin
  std::vector<std::vector<int32_t>> bin_groups(static_cast<size_t>(nb));
  typedef std::pair<int64_t, int64_t> Key;
  std::priority_queue<Key, std::vector<Key>, std::greater<Key>> heap;
  for (int64_t i = 0; i < nb; ++i) heap.push({0, i});
  for (size_t gi = 0; gi < groups.size(); ++gi) {
    const Key k = heap.top();
    heap.pop();
    bin_groups[static_cast<size_t>(k.second)].push_back(static_cast<int32_t>(gi));
    heap.push({k.first + groups[gi].cost, k.second});
  }
  // each bin's groups to its items, first fit
  struct Item {
    int units = 0;
    std::vector<int32_t> members;   // group indices, in the order placed
  };
  std::vector<std::vector<Item>> bin_items(static_cast<size_t>(nb));
  int64_t total = 0;
  for (int64_t b = 0; b < nb; ++b) {
    std::vector<Item>& items = bin_items[static_cast<size_t>(b)];
    for (int32_t gi : bin_groups[static_cast<size_t>(b)]) {
      const Group& g = groups[static_cast<size_t>(gi)];
      size_t k = 0;
      while (k < items.size() && items[k].units + g.units > ucap) ++k;
      if (k == items.size()) items.emplace_back();
      items[k].units += g.units;
      items[k].members.push_back(gi);
    }
    total += static_cast<int64_t>(items.size());
  }
  const int64_t ints = total * pakv::kItemInts;
  if (ints > capacity) return PA_ERR_INVALID;
  int64_t extra = nb;   // index of the next item listed after the first ones
  for (int64_t b = 0; b < nb; ++b) {
    const std::vector<Item>& items = bin_items[static_cast<size_t>(b)];
    int64_t idx = b;
    for (size_t k = 0; k < items.size(); ++k) {
      const int64_t nxt = k + 1 < items.size() ? extra++ : 0;
      int32_t* it = plan + idx * pakv::kItemInts;
      for (int j = 0; j < pakv::kItemInts; ++j) it[j] = j < pakv::kItemUnits ? -1 : 0;
      int u = 0;
      int64_t before = 0;
      uint32_t rot = 0;
      for (int32_t gi : items[k].members) {
        const Group& g = groups[static_cast<size_t>(gi)];
        const int64_t n = std::min<int64_t>(std::max(context_lens_host[g.b], 0), max_tok);
        const int64_t pages = (n + pakv::kPage - 1) / pakv::kPage;
        for (int32_t j = 0; j < g.units; ++j, ++u) {
          const int64_t s = g.s0 + j;
          it[u] = static_cast<int32_t>(static_cast<uint32_t>(g.b) | (static_cast<uint32_t>(s) << 20));
          rot |= static_cast<uint32_t>(before % W) << (4 * u);
          before += pages > 0 ? split_pairs(pages, s) : 0;
        }
      }
      it[pakv::kItemUnits] = static_cast<int32_t>(rot);
      it[pakv::kItemUnits + 1] = static_cast<int32_t>(nxt);
      idx = nxt;
    }
  }
  *num_ints = static_cast<int32_t>(ints);
  return PA_OK;
}

pa_status pa_decode_planned(const pa_pool* pool, const void* q, int32_t num_seqs,
                            int32_t num_q_heads, const int32_t* block_tables,
                            int32_t max_pages_per_seq, const int32_t* context_lens, float scale,
                            float* out, void* workspace, size_t workspace_bytes,
                            const int32_t* plan, int32_t num_ints, void* stream) {
  if (!pool) return PA_ERR_NULL;
  if (!plan && num_seqs > 0) return PA_ERR_NULL;
  return decode_impl(pool, q, num_seqs, num_q_heads, block_tables, max_pages_per_seq, context_lens, scale, out,
                     workspace, workspace_bytes, plan, nullptr, num_ints, stream);
}

pa_status pa_decode_planned_host(const pa_pool* pool, const void* q, int32_t num_seqs, int32_t num_q_heads,
                                 const int32_t* block_tables, int32_t max_pages_per_seq,
                                 const int32_t* context_lens, float scale, float* out, void* workspace,
                                 size_t workspace_bytes, const int32_t* plan_host, int32_t num_ints,
                                 void* stream) {
  if (!pool) return PA_ERR_NULL;
  if (!plan_host && num_seqs > 0) return PA_ERR_NULL;
  return decode_impl(pool, q, num_seqs, num_q_heads, block_tables, max_pages_per_seq, context_lens, scale, out,
                     workspace, workspace_bytes, nullptr, plan_host, num_ints, stream);
}

pa_status pa_decode_static(const pa_pool* pool, const void* q, int32_t num_seqs, int32_t num_q_heads,
                           const int32_t* block_tables, int32_t max_pages_per_seq,
                           const int32_t* context_lens, float scale, float* out, void* stream) {
  if (!pool) return PA_ERR_NULL;
  if (num_seqs < 0 || num_q_heads < 1 || max_pages_per_seq < 1) return PA_ERR_INVALID;
  if (num_q_heads % pool->num_kv_heads != 0) return PA_ERR_INVALID;
  if (num_seqs == 0) return PA_OK;
  size_t acc_bytes = 0, need = 0;
  workspace_parts(pool->head_dim, num_seqs, num_q_heads, num_q_heads / pool->num_kv_heads, max_pages_per_seq,
                  &acc_bytes, &need);
  if (need > kStaticScratchBytes) return PA_ERR_WORKSPACE;
  void* ws = nullptr;
  const pa_status st = static_scratch(&ws);
  if (st != PA_OK) return st;
  return decode_impl(pool, q, num_seqs, num_q_heads, block_tables, max_pages_per_seq, context_lens, scale, out,
                     ws, kStaticScratchBytes, nullptr, nullptr, 0, stream);
}

pa_status pa_decode_append(const pa_pool* pool, const void* q, const void* k_new, const void* v_new,
                           const int32_t* positions, int32_t num_seqs, int32_t num_q_heads,
                           const int32_t* block_tables, int32_t max_pages_per_seq,
                           const int32_t* context_lens, float scale, float* out, void* workspace,
                           size_t workspace_bytes, void* stream) {
  // every argument of both halves is checked before either is queued
  if (!pool) return PA_ERR_NULL;
  if (num_seqs < 0 || num_q_heads < 1 || max_pages_per_seq < 1) return PA_ERR_INVALID;
  if (static_cast<int64_t>(max_pages_per_seq) * pakv::kPage > INT_MAX) return PA_ERR_INVALID;
  if (!scale_ok(scale)) return PA_ERR_INVALID;
  if (num_q_heads % pool->num_kv_heads != 0) return PA_ERR_INVALID;
  const int group = num_q_heads / pool->num_kv_heads;
  if (group > kMaxGroup) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PA_OK;
  if (!q || !block_tables || !context_lens || !out || !k_new || !v_new || !positions) return PA_ERR_NULL;
  if (!aligned16(q) || !aligned4(block_tables) || !aligned4(context_lens) || !aligned16(out) ||
      !aligned16(k_new) || !aligned16(v_new) || !aligned4(positions))
    return PA_ERR_ALIGN;
  size_t acc_bytes = 0, need = 0;
  workspace_parts(pool->head_dim, num_seqs, num_q_heads, group, max_pages_per_seq, &acc_bytes, &need);
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return PA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return PA_ERR_ALIGN;
  }
  pa_status st = pa_kv_append(pool, k_new, v_new, num_seqs, block_tables, max_pages_per_seq, positions, stream);
  if (st != PA_OK) return st;
  return decode_impl(pool, q, num_seqs, num_q_heads, block_tables, max_pages_per_seq, context_lens, scale, out,
                     workspace, workspace_bytes, nullptr, nullptr, 0, stream);
}

// Shared validation of a chunked (prefill / chunk write) call.
static pa_status check_chunk_args(const pa_pool* pool, int32_t num_seqs, int32_t num_rows,
                                  int32_t max_chunk, const int32_t* query_start,
                                  const int32_t* block_tables, int32_t max_pages_per_seq,
                                  const int32_t* context_lens) {
  if (!pool) return PA_ERR_NULL;
  if (num_seqs < 0 || num_rows < 0 || max_chunk < 0 || max_pages_per_seq < 1) return PA_ERR_INVALID;
  if (static_cast<int64_t>(max_pages_per_seq) * pakv::kPage > INT_MAX) return PA_ERR_INVALID;
  if (num_seqs == 0 || num_rows == 0 || max_chunk == 0) return PA_OK;
  if (!query_start || !block_tables || !context_lens) return PA_ERR_NULL;
  if (!aligned4(query_start) || !aligned4(block_tables) || !aligned4(context_lens)) return PA_ERR_ALIGN;
  return PA_OK;
}

static pa_status launch_write(const pa_pool* pool, const void* k_rows, const void* v_rows,
                              int32_t num_seqs, int32_t num_rows, int32_t max_chunk,
                              const int32_t* query_start, const int32_t* block_tables,
                              int32_t max_pages_per_seq, const int32_t* context_lens,
                              hipStream_t s) {
  pakv::WriteArgs a;
  a.kpool = static_cast<uint16_t*>(pool->k);
  a.vpool = static_cast<uint16_t*>(pool->v);
  a.k_rows = static_cast<const uint16_t*>(k_rows);
  a.v_rows = static_cast<const uint16_t*>(v_rows);
  a.query_start = query_start;
  a.block_tables = block_tables;
  a.ctx_before = context_lens;
  a.num_pages = pool->num_pages;
  a.num_seqs = num_seqs;
  a.num_rows = num_rows;
  a.num_kv_heads = pool->num_kv_heads;
  a.stride = max_pages_per_seq;
  a.max_chunk = max_chunk;
  a.pages_per_seq = (max_chunk + pakv::kPage - 1) / pakv::kPage + 1;
  const int64_t blocks = static_cast<int64_t>(num_seqs) * a.pages_per_seq;
  if (blocks > INT_MAX) return PA_ERR_INVALID;
  (void)hipGetLastError();
  {
    LaunchTimer t(3, s);
    if (pool->head_dim == 64)
      hipLaunchKernelGGL((pakv::kv_write_kernel<64>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((pakv::kv_write_kernel<128>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, a);
  }
  if (hipGetLastError() != hipSuccess) return PA_ERR_LAUNCH;
  return PA_OK;
}

pa_status pa_kv_write(const pa_pool* pool, const void* k_rows, const void* v_rows, int32_t num_seqs,
                      int32_t num_rows, int32_t max_chunk, const int32_t* query_start,
                      const int32_t* block_tables, int32_t max_pages_per_seq,
                      const int32_t* context_lens, void* stream) {
  pa_status st = check_chunk_args(pool, num_seqs, num_rows, max_chunk, query_start, block_tables,
                                  max_pages_per_seq, context_lens);
  if (st != PA_OK || num_seqs == 0 || num_rows == 0 || max_chunk == 0) return st;
  if (!k_rows || !v_rows) return PA_ERR_NULL;
  if (!aligned16(k_rows) || !aligned16(v_rows)) return PA_ERR_ALIGN;
  return launch_write(pool, k_rows, v_rows, num_seqs, num_rows, max_chunk, query_start, block_tables,
                      max_pages_per_seq, context_lens, static_cast<hipStream_t>(stream));
}

// Row blocks per (sequence, KV head) for chunks of up to max_chunk tokens.
static int64_t prefill_row_blocks(int d, int64_t max_chunk, int group) {
  const int block_rows = d == 64 ? pakv::prefill_block_rows<64>() : pakv::prefill_block_rows<128>();
  return (max_chunk * group + block_rows - 1) / block_rows;
}

static pa_status prefill_impl(const pa_pool* pool, const void* q, const void* k_rows, const void* v_rows,
                              int32_t num_seqs, int32_t num_q_heads, int32_t num_rows, int32_t max_chunk,
                              const int32_t* query_start, const int32_t* block_tables,
                              int32_t max_pages_per_seq, const int32_t* context_lens, float scale,
                              float* out, const int32_t* plan, int32_t plan_items, void* stream) {
  pa_status st = check_chunk_args(pool, num_seqs, num_rows, max_chunk, query_start, block_tables,
                                  max_pages_per_seq, context_lens);
  if (st != PA_OK) return st;
  if (num_q_heads < 1 || num_q_heads % pool->num_kv_heads != 0) return PA_ERR_INVALID;
  if (!scale_ok(scale)) return PA_ERR_INVALID;
  const int group = num_q_heads / pool->num_kv_heads;
  if (group > kMaxGroup) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0 || num_rows == 0 || max_chunk == 0) return PA_OK;
  if (!q || !k_rows || !v_rows || !out) return PA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_rows) || !aligned16(v_rows) || !aligned16(out)) return PA_ERR_ALIGN;
  const int64_t row_blocks = prefill_row_blocks(pool->head_dim, max_chunk, group);
  if (plan) {
    if (num_seqs > kPlanMaxSeqs || row_blocks > kPlanMaxSplits) return PA_ERR_INVALID;
    if (!aligned4(plan)) return PA_ERR_ALIGN;
  }
  if (plan_items < 0 || plan_items > static_cast<int64_t>(num_seqs) * row_blocks) return PA_ERR_INVALID;
  if (plan_items > 0 && !plan) return PA_ERR_NULL;
  const int64_t units = plan ? plan_items : static_cast<int64_t>(num_seqs) * row_blocks;
  const int64_t blocks = static_cast<int64_t>(pool->num_kv_heads) * units;
  if (blocks > INT_MAX || row_blocks > INT_MAX) return PA_ERR_INVALID;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = launch_write(pool, k_rows, v_rows, num_seqs, num_rows, max_chunk, query_start, block_tables,
                    max_pages_per_seq, context_lens, s);
  if (st != PA_OK || blocks == 0) return st;
  pakv::PrefillArgs a;
  a.kpool = static_cast<const uint16_t*>(pool->k);
  a.vpool = static_cast<const uint16_t*>(pool->v);
  a.q = static_cast<const uint16_t*>(q);
  a.query_start = query_start;
  a.block_tables = block_tables;
  a.ctx_before = context_lens;
  a.out = out;
  a.num_pages = pool->num_pages;
  a.num_seqs = num_seqs;
  a.num_rows = num_rows;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = pool->num_kv_heads;
  a.group = group;
  a.stride = max_pages_per_seq;
  a.max_chunk = max_chunk;
  a.row_blocks = static_cast<int32_t>(row_blocks);
  a.scale_log2 = scale_log2_of(scale);
  a.plan = plan;
  (void)hipGetLastError();
  {
    LaunchTimer t(4, s);
    if (pool->head_dim == 64)
      hipLaunchKernelGGL((pakv::prefill_kernel<64>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((pakv::prefill_kernel<128>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, a);
  }
  if (hipGetLastError() != hipSuccess) return PA_ERR_LAUNCH;
  return PA_OK;
}

pa_status pa_prefill(const pa_pool* pool, const void* q, const void* k_rows, const void* v_rows,
                     int32_t num_seqs, int32_t num_q_heads, int32_t num_rows, int32_t max_chunk,
                     const int32_t* query_start, const int32_t* block_tables,
                     int32_t max_pages_per_seq, const int32_t* context_lens, float scale,
                     float* out, void* stream) {
  return prefill_impl(pool, q, k_rows, v_rows, num_seqs, num_q_heads, num_rows, max_chunk, query_start,
                      block_tables, max_pages_per_seq, context_lens, scale, out, nullptr, 0, stream);
}

int64_t pa_prefill_plan_capacity(const pa_pool* pool, int32_t num_seqs, int32_t num_q_heads,
                                 int32_t max_chunk) {
  if (!pool || num_seqs < 0 || num_q_heads < 1 || max_chunk < 0) return -1;
  if (num_q_heads % pool->num_kv_heads != 0) return -1;
  const int group = num_q_heads / pool->num_kv_heads;
  if (group > kMaxGroup) return -1;
  const int64_t row_blocks = prefill_row_blocks(pool->head_dim, max_chunk, group);
  if (num_seqs > kPlanMaxSeqs || row_blocks > kPlanMaxSplits) return -1;
  return static_cast<int64_t>(num_seqs) * row_blocks;
}

static pa_status prefill_plan_impl(const pa_pool* pool, const int32_t* context_lens_host,
                                   const int32_t* chunk_lens_host, int32_t num_seqs, int32_t num_q_heads,
                                   int32_t max_pages_per_seq, int32_t max_chunk, int32_t* plan,
                                   int64_t capacity, int32_t* num_items);

pa_status pa_prefill_plan(const pa_pool* pool, const int32_t* context_lens_host,
                          const int32_t* chunk_lens_host, int32_t num_seqs, int32_t num_q_heads,
                          int32_t max_pages_per_seq, int32_t max_chunk, int32_t* plan,
                          int64_t capacity, int32_t* num_items) {
  if (!pool || !num_items) return PA_ERR_NULL;
  *num_items = 0;
  if (max_pages_per_seq < 1) return PA_ERR_INVALID;
  if (static_cast<int64_t>(max_pages_per_seq) * pakv::kPage > INT_MAX) return PA_ERR_INVALID;
  if (pa_prefill_plan_capacity(pool, num_seqs, num_q_heads, max_chunk) < 0) return PA_ERR_INVALID;
  if (num_seqs == 0 || max_chunk == 0) return PA_OK;
  if (!context_lens_host || !chunk_lens_host || !plan) return PA_ERR_NULL;
  try {
    return prefill_plan_impl(pool, context_lens_host, chunk_lens_host, num_seqs, num_q_heads,
                             max_pages_per_seq, max_chunk, plan, capacity, num_items);
  } catch (...) {   // out of host memory; nothing escapes the C ABI
    *num_items = 0;
    return PA_ERR_INVALID;
  }
}

static pa_status prefill_plan_impl(const pa_pool* pool, const int32_t* context_lens_host,
                                   const int32_t* chunk_lens_host, int32_t num_seqs, int32_t num_q_heads,
                                   int32_t max_pages_per_seq, int32_t max_chunk, int32_t* plan,
                                   int64_t capacity, int32_t* num_items) {
  const int d = pool->head_dim;
  const int group = num_q_heads / pool->num_kv_heads;
  const int block_rows = d == 64 ? pakv::prefill_block_rows<64>() : pakv::prefill_block_rows<128>();
  const int64_t row_blocks = prefill_row_blocks(d, max_chunk, group);
  const int64_t max_tok = static_cast<int64_t>(max_pages_per_seq) * pakv::kPage;
  // every row block that holds rows, with the page pairs its rows can see
  // (the kernel's own clamping of the cache and chunk lengths), visited from
  // the last row block down and in sequence order, as the unplanned grid
  struct Item {
    int64_t pairs;
    uint32_t code;
  };
  std::vector<Item> items;
  for (int64_t rb = row_blocks - 1; rb >= 0; --rb) {
    for (int32_t b = 0; b < num_seqs; ++b) {
      const int64_t c = std::min<int64_t>(std::max(context_lens_host[b], 0), max_tok);
      int64_t n = std::min<int64_t>(std::max(chunk_lens_host[b], 0), max_chunk);
      n = std::min(n, max_tok - c);
      const int64_t rows = n * group;
      if (rb * block_rows >= rows) continue;
      const int64_t last_pos = c + std::min<int64_t>(rb * block_rows + block_rows - 1, rows - 1) / group;
      const int64_t pages = (last_pos + pakv::kPage) / pakv::kPage;
      items.push_back({(pages + 1) / 2, static_cast<uint32_t>(b) | (static_cast<uint32_t>(rb) << 20)});
    }
  }
  if (static_cast<int64_t>(items.size()) > capacity) return PA_ERR_INVALID;
  std::stable_sort(items.begin(), items.end(), [](const Item& x, const Item& y) { return x.pairs > y.pairs; });
  const int64_t total = static_cast<int64_t>(items.size());
  for (int64_t i = 0; i < total; ++i) plan[i] = static_cast<int32_t>(items[i].code);
  // A grid the device holds at once: each CU takes the items of one tier
  // position of its XCD (XCD round-robin over workgroups, KV head fastest,
  // then the XCD's CUs in order); reversing every other tier pairs the large
  // items with small ones on each CU.
  const int hkv = pool->num_kv_heads;
  const int64_t resident = static_cast<int64_t>(kDeviceCUs) * prefill_wgs_per_cu(d);
  const int64_t tier = (hkv <= 8 && 8 % hkv == 0) ? kCUsPerXCD * (8 / hkv) : kCUsPerXCD;
  if (total * hkv <= resident) {
    for (int64_t t0 = tier; t0 < total; t0 += 2 * tier)
      std::reverse(plan + t0, plan + std::min<int64_t>(t0 + tier, total));
  }
  *num_items = static_cast<int32_t>(total);
  return PA_OK;
}

pa_status pa_prefill_planned(const pa_pool* pool, const void* q, const void* k_rows,
                             const void* v_rows, int32_t num_seqs, int32_t num_q_heads,
                             int32_t num_rows, int32_t max_chunk, const int32_t* query_start,
                             const int32_t* block_tables, int32_t max_pages_per_seq,
                             const int32_t* context_lens, float scale, float* out,
                             const int32_t* plan, int32_t num_items, void* stream) {
  if (!pool) return PA_ERR_NULL;
  if (!plan && num_items > 0) return PA_ERR_NULL;
  return prefill_impl(pool, q, k_rows, v_rows, num_seqs, num_q_heads, num_rows, max_chunk, query_start,
                      block_tables, max_pages_per_seq, context_lens, scale, out, plan, num_items, stream);
}

pa_status pa_profile_start(void) {
  for (auto& r : g_records) {
    g_free_events.push_back(r.start);
    g_free_events.push_back(r.stop);
  }
  g_records.clear();
  g_profiling = true;
  return PA_OK;
}

pa_status pa_profile_stop(double* ms, int64_t* launches) {
  if (!ms || !launches) return PA_ERR_NULL;
  g_profiling = false;
  for (int k = 0; k < kProfileKinds; ++k) {
    ms[k] = 0.0;
    launches[k] = 0;
  }
  pa_status st = PA_OK;
  for (auto& r : g_records) {
    if (hipEventSynchronize(r.stop) != hipSuccess) {
      st = PA_ERR_LAUNCH;
      continue;
    }
    float t = 0.f;
    if (hipEventElapsedTime(&t, r.start, r.stop) != hipSuccess) {
      st = PA_ERR_LAUNCH;
      continue;
    }
    ms[r.kind] += t;
    launches[r.kind] += 1;
  }
  for (auto& r : g_records) {
    g_free_events.push_back(r.start);
    g_free_events.push_back(r.stop);
  }
  g_records.clear();
  return st;
}

pa_status pa_stream_read(const void* src, size_t bytes, void* sink, void* stream) {
  if (!src || !sink) return PA_ERR_NULL;
  if (bytes == 0 || bytes % 16 != 0) return PA_ERR_INVALID;
  if (!aligned16(src) || !aligned16(sink)) return PA_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  hipLaunchKernelGGL(pakv::stream_read_kernel, dim3(16384), dim3(256), 0, s,
                     static_cast<const pakv::u32x4*>(src), bytes / 16, static_cast<uint32_t*>(sink));
  if (hipGetLastError() != hipSuccess) return PA_ERR_LAUNCH;
  return PA_OK;
}

}  // extern "C"
