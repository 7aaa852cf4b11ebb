// Host planner: request lengths -> one work list for the fused POD grid.
//
// It follows what the POD article (www.dpshk.com/news/5405057) says plan() does
// ("plan 内部做了什么", "Batch 版本 plan 的 colocated-CTA 调度细节"): read the
// host copies of the length arrays, derive each request's KV length from its
// page count and last_page_len, split decode KV into chunks (split-KV), and
// decide how prefill and decode work share the device. Our version emits one
// list of workgroup items for both roles instead of two kernel plans, and
// places items on the MI355X's accelerator dies explicitly.
#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdio>
#include <string>
#include <vector>

#include "pod_internal.h"

namespace pod {

namespace {

struct Item {
  int32_t w[kItemWords];
  int64_t cost;
  int32_t xcd;
};

struct Req {
  int role;
  int b;
  int32_t qo_start, qo_len, kv_len, page_start;
};

int fail(std::string* err, int code, const std::string& msg) {
  if (err) *err = msg;
  return code;
}

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Cost estimates used only to place and order items, in nanoseconds of one
// persistent workgroup (one CU) on MI355X: a query tile streams 64-key blocks at
// ~2.1 us each (~33 ns per key) plus ~1.5 us at its boundary (output store and
// the next tile's query load); a key chunk moves 512 bytes per key at ~20 ns per
// key plus ~2.5 us to start its load pipeline. Measured per item.
constexpr int64_t kTileCostPerKey = 33;
constexpr int64_t kTileCostFixed = 1500;
constexpr int64_t kChunkCostPerKey = 20;
constexpr int64_t kChunkCostFixed = 2500;
// Share of the key chunks' estimated cost left to a shared queue that the
// workgroups drain once their own lists are done: it absorbs what the estimates
// miss (dies and CUs do not all stream HBM at the same rate).
// A tenth measured best on the pod step (2 x 2048 prefill + 128 decodes on
// 2048 keys: ~9 us faster than a quarter, same-box A/B); decode alone and the
// chunked-prefill step do not change.
constexpr double kPoolShare = 0.10;

int validate_role(const pod_role_desc& r, const char* name, int page_size, std::string* err) {
  char buf[256];
  if (r.batch < 0) {
    snprintf(buf, sizeof buf, "%s.batch must be >= 0", name);
    return fail(err, POD_ERR_INVALID, buf);
  }
  if (r.batch == 0) return POD_OK;
  // the kernels keep scores times scale_log2 in fp32 next to a -1e30 start
  // value; scales beyond 1e6 (or NaN) are refused
  if (!(r.sm_scale <= 1e6f)) {
    snprintf(buf, sizeof buf, "%s.sm_scale must be <= 1e6", name);
    return fail(err, POD_ERR_INVALID, buf);
  }
  if (!r.qo_indptr || !r.kv_indptr || !r.last_page_len) {
    snprintf(buf, sizeof buf, "%s: qo_indptr, kv_indptr and last_page_len are required", name);
    return fail(err, POD_ERR_INVALID, buf);
  }
  if (r.qo_indptr[0] != 0 || r.kv_indptr[0] != 0) {
    snprintf(buf, sizeof buf, "%s: qo_indptr[0] and kv_indptr[0] must be 0", name);
    return fail(err, POD_ERR_INVALID, buf);
  }
  if (r.window_left < -1) {
    snprintf(buf, sizeof buf, "%s.window_left must be -1 or >= 0", name);
    return fail(err, POD_ERR_INVALID, buf);
  }
  for (int b = 0; b < r.batch; ++b) {
    int64_t q0 = r.qo_indptr[b], q1 = r.qo_indptr[b + 1];
    int64_t p0 = r.kv_indptr[b], p1 = r.kv_indptr[b + 1];
    if (q1 < q0) {
      snprintf(buf, sizeof buf, "%s: qo_indptr decreases at request %d", name, b);
      return fail(err, POD_ERR_INVALID, buf);
    }
    if (p1 <= p0) {
      snprintf(buf, sizeof buf, "%s: request %d holds no page (kv_indptr must increase)", name, b);
      return fail(err, POD_ERR_INVALID, buf);
    }
    int32_t lpl = r.last_page_len[b];
    if (lpl < 1 || lpl > page_size) {
      snprintf(buf, sizeof buf, "%s: last_page_len[%d] = %d outside [1, page_size=%d]", name, b,
               lpl, page_size);
      return fail(err, POD_ERR_INVALID, buf);
    }
    int64_t kv_len = (p1 - p0 - 1) * (int64_t)page_size + lpl;
    if (kv_len > INT32_MAX / 2) {
      snprintf(buf, sizeof buf, "%s: request %d kv_len too large", name, b);
      return fail(err, POD_ERR_INVALID, buf);
    }
    if (r.causal && kv_len < q1 - q0) {
      snprintf(buf, sizeof buf, "%s: causal request %d has kv_len %lld < q_len %lld", name, b,
               (long long)kv_len, (long long)(q1 - q0));
      return fail(err, POD_ERR_INVALID, buf);
    }
  }
  return POD_OK;
}

}  // namespace

int plan_compute(const pod_plan_desc& d, const ImageSink& sink, pod_plan_info& info,
                 std::string* err, bool fixed_grid) {
  info = pod_plan_info{};
  if (d.num_qo_heads <= 0 || d.num_kv_heads <= 0)
    return fail(err, POD_ERR_INVALID, "num_qo_heads and num_kv_heads must be positive");
  if (d.num_qo_heads % d.num_kv_heads)
    return fail(err, POD_ERR_INVALID, "num_qo_heads must be a multiple of num_kv_heads");
  if (d.head_dim != kHeadDim) return fail(err, POD_ERR_UNSUPPORTED, "head_dim must be 128");
  if (d.page_size < 1) return fail(err, POD_ERR_INVALID, "page_size must be >= 1");
  if (d.dtype != POD_DTYPE_F16 && d.dtype != POD_DTYPE_BF16)
    return fail(err, POD_ERR_UNSUPPORTED, "dtype must be POD_DTYPE_F16 or POD_DTYPE_BF16");
  if (d.order < 0 || d.order > 3) return fail(err, POD_ERR_INVALID, "unknown order policy");
  const int g = d.num_qo_heads / d.num_kv_heads;
  if (g > kMaxGroup) return fail(err, POD_ERR_UNSUPPORTED, "group size above 128 is not supported");
  if (d.num_kv_heads > kMaxKvHeads) return fail(err, POD_ERR_UNSUPPORTED, "more than 16384 kv heads");
  if (d.has_sinks && d.num_qo_heads > kMaxSinkHeads)
    return fail(err, POD_ERR_UNSUPPORTED, "sinks with more than 1024 qo heads are not supported");
  int rc = validate_role(d.prefill, "prefill", d.page_size, err);
  if (rc) return rc;
  rc = validate_role(d.decode, "decode", d.page_size, err);
  if (rc) return rc;
  const int num_cus = d.num_cus > 0 ? d.num_cus : 256;   // >= 1
  const int H = d.num_kv_heads;

  // per-request table: prefill requests first, then decode requests
  std::vector<Req> reqs;
  const pod_role_desc* roles[2] = {&d.prefill, &d.decode};
  for (int role = 0; role < 2; ++role) {
    const pod_role_desc& r = *roles[role];
    for (int b = 0; b < r.batch; ++b) {
      Req q;
      q.role = role;
      q.b = b;
      q.qo_start = r.qo_indptr[b];
      q.qo_len = r.qo_indptr[b + 1] - r.qo_indptr[b];
      q.kv_len = (r.kv_indptr[b + 1] - r.kv_indptr[b] - 1) * d.page_size + r.last_page_len[b];
      q.page_start = r.kv_indptr[b];
      reqs.push_back(q);
    }
  }

  // key range a request's rows need as a whole: [lo, kv_len)
  auto chunk_lo = [&](const Req& q) -> int64_t {
    const pod_role_desc& r = *roles[q.role];
    int64_t p0 = (int64_t)q.kv_len - q.qo_len;
    return r.window_left >= 0 ? std::max<int64_t>(0, p0 - r.window_left) : 0;
  };
  if (d.decode_kv_dtype != 0 && d.decode_kv_dtype != d.dtype && d.decode_kv_dtype != POD_DTYPE_FP8_E4M3)
    return fail(err, POD_ERR_UNSUPPORTED, "decode_kv_dtype must be 0, dtype or POD_DTYPE_FP8_E4M3");
  const bool fp8_d = d.decode_kv_dtype == POD_DTYPE_FP8_E4M3;
  // Key chunks hold up to 32 rows (q_len x group) of one (request, kv head).
  // Requests with more rows run as query tiles, except on an FP8 decode cache
  // (its bytes are widened as a key chunk stages them): those are cut into row
  // slices of 32, each a key chunk of its own over the same keys.
  auto is_chunk = [&](const Req& q) {
    return (int64_t)q.qo_len * g <= kChunkRows || (q.role == 1 && fp8_d);
  };
  auto n_slices = [&](const Req& q) -> int64_t {
    return ((int64_t)q.qo_len * g + kChunkRows - 1) / kChunkRows;
  };

  // decode split size: enough key-chunk items for ~4 per CU, at least 256 keys each
  int64_t chunk_keys_total = 0;
  for (const Req& q : reqs)
    if (q.qo_len > 0 && is_chunk(q)) chunk_keys_total += (int64_t)H * n_slices(q) * (q.kv_len - chunk_lo(q));
  int64_t C;
  if (d.decode_chunk < 0) {
    C = INT32_MAX;
  } else if (d.decode_chunk > 0) {
    C = round_up(d.decode_chunk, 64);
  } else {
    int64_t target = 4LL * num_cus;
    C = std::max<int64_t>(256, round_up((chunk_keys_total + target - 1) / std::max<int64_t>(target, 1), 64));
  }

  // exact item count first, so the item array is allocated once
  const int T = std::max(1, kTileRows / g);
  size_t n_items_total = 0;
  for (const Req& q : reqs) {
    if (q.qo_len == 0) continue;
    if (is_chunk(q)) n_items_total += (size_t)H * (size_t)n_slices(q) * (size_t)((q.kv_len - chunk_lo(q) + C - 1) / C);
    else n_items_total += (size_t)H * (size_t)((q.qo_len + T - 1) / T);
  }
  std::vector<Item> items(n_items_total);
  std::vector<int32_t> groups;  // n_groups x 4
  groups.reserve(n_items_total * kGroupWords);
  int32_t n_slots = 0;
  size_t ni = 0;
  for (size_t ri = 0; ri < reqs.size(); ++ri) {
    const Req& q = reqs[ri];
    const pod_role_desc& r = *roles[q.role];
    if (q.qo_len == 0) continue;
    if (is_chunk(q)) {
      const int64_t lo = chunk_lo(q), hi = q.kv_len;
      const int64_t splits = (hi - lo + C - 1) / C;
      const int64_t ns = n_slices(q);
      for (int kvh = 0; kvh < H; ++kvh) {
        // one split group per row slice; a key range's slices are consecutive items
        const int32_t grp0 = splits > 1 ? (int32_t)(groups.size() / kGroupWords) : -1;
        if (splits > 1)
          for (int64_t sl = 0; sl < ns; ++sl) {
            groups.push_back((int32_t)splits);
            groups.push_back(n_slots);
            groups.push_back((int32_t)ri);
            groups.push_back(kvh);
            n_slots += (int32_t)splits;
          }
        for (int64_t sp = 0; sp < splits; ++sp)
          for (int64_t sl = 0; sl < ns; ++sl) {
            const int32_t grp = splits > 1 ? grp0 + (int32_t)sl : -1;
            Item& it = items[ni++];
            const int64_t b0 = lo + sp * C, b1 = std::min<int64_t>(hi, b0 + C);
            it.w[0] = q.role | kFlagChunk | (int32_t)(sp << kSplitShift);
            it.w[1] = (int32_t)ri;
            it.w[2] = kvh;
            it.w[3] = (int32_t)(sl * kChunkRows);   // first row (token x group) of the slice
            it.w[4] = q.qo_len;
            it.w[5] = (int32_t)b0;
            it.w[6] = (int32_t)b1;
            it.w[7] = grp;
            it.cost = kChunkCostFixed + kChunkCostPerKey * (b1 - b0);
            it.xcd = -1;
          }
      }
    } else {
      for (int t0 = 0; t0 < q.qo_len; t0 += T) {
        const int ntok = std::min(T, q.qo_len - t0);
        const int64_t pf = (int64_t)q.kv_len - q.qo_len + t0, pl = pf + ntok - 1;
        const int64_t hi = r.causal ? pl + 1 : q.kv_len;
        const int64_t lo = r.window_left >= 0 ? std::max<int64_t>(0, pf - r.window_left) : 0;
        for (int kvh = 0; kvh < H; ++kvh) {
          Item& it = items[ni++];
          it.w[0] = q.role;
          it.w[1] = (int32_t)ri;
          it.w[2] = kvh;
          it.w[3] = t0;
          it.w[4] = ntok;
          it.w[5] = (int32_t)lo;
          it.w[6] = (int32_t)hi;
          it.w[7] = -1;
          it.cost = kTileCostFixed + kTileCostPerKey * (hi - lo);
          // tiles sharing one request's K/V for one kv head stay on one die (L2 reuse)
          it.xcd = (int32_t)((ri * (size_t)H + kvh) % kNumXcds);
        }
      }
    }
  }

  // Heaviest first: a stable counting sort on the cost quantised to 1024 levels.
  int64_t max_cost = 1, total_cost = 0, max_tile_cost = 0;
  for (const Item& it : items) {
    max_cost = std::max(max_cost, it.cost);
    total_cost += it.cost;
    if (!(it.w[0] & kFlagChunk)) max_tile_cost = std::max(max_tile_cost, it.cost);
  }
  constexpr int kLevels = 1024;
  std::vector<int32_t> bucket_start(kLevels + 1, 0);
  std::vector<int16_t> level(items.size());
  const double to_level = (double)(kLevels - 1) / (double)max_cost;
  for (size_t i = 0; i < items.size(); ++i) {
    // level 0 = heaviest
    const int lv = std::min(kLevels - 1, (int)((double)(max_cost - items[i].cost) * to_level));
    level[i] = (int16_t)lv;
    ++bucket_start[lv + 1];
  }
  for (int b = 0; b < kLevels; ++b) bucket_start[b + 1] += bucket_start[b];
  std::vector<uint32_t> order(items.size());
  for (size_t i = 0; i < items.size(); ++i) order[bucket_start[level[i]]++] = (uint32_t)i;

  // Dies. The query tiles of one (request, kv head) unit share its K/V, so a
  // unit gets a home die (units heaviest first onto the least loaded die) and
  // its tiles go there unless that die would pass an even share of all work by
  // more than one tile (few large units then still spread over every die).
  // Key chunks then fill the least loaded dies, heaviest first.
  int64_t load[kNumXcds] = {};
  {
    std::vector<int64_t> unit_cost(reqs.size() * (size_t)H, 0);
    for (const Item& it : items)
      if (!(it.w[0] & kFlagChunk)) unit_cost[(size_t)it.w[1] * H + it.w[2]] += it.cost;
    std::vector<uint32_t> units;
    for (size_t u = 0; u < unit_cost.size(); ++u)
      if (unit_cost[u] > 0) units.push_back((uint32_t)u);
    std::stable_sort(units.begin(), units.end(),
                     [&](uint32_t x, uint32_t y) { return unit_cost[x] > unit_cost[y]; });
    std::vector<int8_t> home(unit_cost.size(), 0);
    int64_t uload[kNumXcds] = {};
    for (uint32_t u : units) {
      int best = 0;
      for (int x = 1; x < kNumXcds; ++x)
        if (uload[x] < uload[best]) best = x;
      home[u] = (int8_t)best;
      uload[best] += unit_cost[u];
    }
    const int64_t cap = (total_cost + kNumXcds - 1) / kNumXcds + max_tile_cost;
    for (uint32_t i : order) {
      Item& it = items[i];
      if (it.w[0] & kFlagChunk) continue;
      int x = home[(size_t)it.w[1] * H + it.w[2]];
      if (load[x] + it.cost > cap) {
        x = 0;
        for (int y = 1; y < kNumXcds; ++y)
          if (load[y] < load[x]) x = y;
      }
      it.xcd = x;
      load[x] += it.cost;
    }
    // key chunks: the least loaded die, heaviest first; the row slices of one
    // (request, kv head, key range) share a die, so all but the first find
    // their K/V in its L2 (the slices of a key range are consecutive items)
    std::vector<uint32_t> pos(items.size());
    for (size_t k = 0; k < order.size(); ++k) pos[order[k]] = (uint32_t)k;
    for (uint32_t i : order) {
      Item& it = items[i];
      if (!(it.w[0] & kFlagChunk)) continue;
      int x = -1;
      if (it.w[3] > 0) {
        // slice 0 of this key range: the item w[3] / 32 places earlier
        const size_t i0 = i - (size_t)(it.w[3] / kChunkRows);
        if (items[i0].xcd >= 0 && pos[i0] < pos[i]) x = items[i0].xcd;
      }
      if (x < 0) {
        x = 0;
        for (int y = 1; y < kNumXcds; ++y)
          if (load[y] < load[x]) x = y;
      }
      it.xcd = x;
      load[x] += it.cost;
    }
  }

  // Workgroups: one per CU; or, when every die's items fit one workgroup each
  // and the grid need not stay fixed, as many per die as the most items a die
  // holds, so a small step launches few idle workgroups.
  int G = num_cus;
  int64_t per_die[kNumXcds] = {};
  for (const Item& it : items) ++per_die[it.xcd];
  const int64_t most = std::max<int64_t>(1, *std::max_element(per_die, per_die + kNumXcds));
  const bool one_each = most * kNumXcds <= num_cus;
  if (!fixed_grid && one_each) G = (int)(most * kNumXcds);
  // The shared pool: the lightest key chunks, up to kPoolShare of their cost
  // (none when every item has a workgroup of its own).
  const bool use_pool = G > 1 && items.size() > (size_t)G;
  std::vector<uint8_t> in_pool(items.size(), 0);
  std::vector<uint32_t> pool;
  {
    int64_t chunk_cost = 0;
    for (const Item& it : items)
      if (it.w[0] & kFlagChunk) chunk_cost += it.cost;
    const int64_t budget = (int64_t)(kPoolShare * (double)chunk_cost);
    int64_t taken = 0;
    for (size_t k = order.size(); k-- > 0 && use_pool;) {   // lightest first
      const Item& it = items[order[k]];
      if (!(it.w[0] & kFlagChunk)) continue;
      if (taken + it.cost > budget) break;
      taken += it.cost;
      in_pool[order[k]] = 1;
    }
    for (uint32_t i : order)   // the queue hands them out heaviest first
      if (in_pool[i]) pool.push_back(i);
  }

  // Workgroups: one persistent workgroup per CU; workgroup w is dispatched to
  // die w % kNumXcds. Each die's items, heaviest first, go to the least loaded
  // of its workgroups (LPT), so every workgroup holds a static list.
  // Per die a min-heap of (load, workgroup); ties go to the lower workgroup.
  std::vector<int32_t> wg_of(items.size(), -1);
  if (one_each) {
    // every die's items fit one workgroup each: the heap below would hand die
    // x's items, in order, to its workgroups x, x + 8, ... (all still empty)
    int32_t next[kNumXcds];
    for (int x = 0; x < kNumXcds; ++x) next[x] = x;
    for (uint32_t i : order) {
      const int x = items[i].xcd;
      wg_of[i] = next[x];
      next[x] += kNumXcds;
    }
  } else {
    using Slot = std::pair<int64_t, int32_t>;
    std::vector<Slot> heap[kNumXcds];
    for (int x = 0; x < kNumXcds; ++x) heap[x].reserve((size_t)(G / kNumXcds + 1));
    for (int w = 0; w < G; ++w) heap[w % kNumXcds].push_back(Slot(0, w));
    auto later = [](const Slot& a, const Slot& b) { return a > b; };
    for (uint32_t i : order) {
      if (in_pool[i]) continue;
      std::vector<Slot>& hp = heap[items[i].xcd < G ? items[i].xcd : items[i].xcd % G];
      std::pop_heap(hp.begin(), hp.end(), later);
      wg_of[i] = hp.back().second;
      hp.back().first += items[i].cost;
      std::push_heap(hp.begin(), hp.end(), later);
    }
  }
  // Each workgroup's list, heaviest first within each kind: prefill-role query
  // tiles, decode-role query tiles (a workgroup runs one block stream per
  // role), then key chunks. One stable counting sort on (workgroup, kind).
  auto kind = [&](const Item& it) { return (it.w[0] & kFlagChunk) ? 2 : (it.w[0] & kFlagRole); };
  std::vector<int32_t> bucket((size_t)G * 3 + 1, 0);
  for (uint32_t i : order)
    if (wg_of[i] >= 0) ++bucket[(size_t)wg_of[i] * 3 + kind(items[i]) + 1];
  for (size_t b = 0; b + 1 < bucket.size(); ++b) bucket[b + 1] += bucket[b];
  std::vector<uint32_t> listed(bucket.back());
  {
    std::vector<int32_t> fill(bucket.begin(), bucket.end() - 1);
    for (uint32_t i : order)
      if (wg_of[i] >= 0) listed[fill[(size_t)wg_of[i] * 3 + kind(items[i])]++] = i;
  }

  // query-tile blocks per workgroup
  int64_t n_blocks = 0;
  for (int w = 0; w < G; ++w) {
    if (bucket[(size_t)w * 3 + 2] - bucket[(size_t)w * 3] >= kMaxTilesPerWg)
      return fail(err, POD_ERR_UNSUPPORTED, "plan too large (query tiles per workgroup)");
  }
  for (uint32_t i : listed)
    if (!(items[i].w[0] & kFlagChunk)) n_blocks += (items[i].w[6] - items[i].w[5] + kTileKeys - 1) / kTileKeys;

  const int n_groups = (int)(groups.size() / kGroupWords);
  const int64_t reqs_off = POD_HDR_WORDS;
  const int64_t items_off = reqs_off + (int64_t)reqs.size() * kReqWords;
  const int64_t tdesc_off = items_off + (int64_t)items.size() * kItemWords;
  const int64_t wgs_off = tdesc_off + (int64_t)items.size() * kTdescWords;
  const int64_t blocks_off = wgs_off + (int64_t)G * kWgWords;
  const int64_t groups_off = blocks_off + n_blocks * kBlockWords;
  const int64_t counters_off = groups_off + (int64_t)n_groups * kGroupWords;
  const int64_t queue_off = counters_off + n_groups;
  const int64_t total = queue_off + 2;
  if (total > INT32_MAX / 2) return fail(err, POD_ERR_UNSUPPORTED, "plan too large");

  info.n_items = (int32_t)items.size();
  info.n_prefill_items = 0;
  for (const Item& it : items) info.n_prefill_items += (it.w[0] & kFlagRole) == 0;
  info.n_decode_items = info.n_items - info.n_prefill_items;
  info.n_groups = n_groups;
  info.n_slots = n_slots;
  info.grid = G;
  info.decode_chunk = (int32_t)std::min<int64_t>(C, INT32_MAX);
  info.image_ints = (int32_t)total;
  info.float_ws_bytes = (int64_t)n_slots * kSlotFloats * 4;
  // two plans alternate between the halves of the int workspace
  info.int_ws_bytes = 2 * ((total * 4 + 255) / 256 * 256);
  int32_t* h = sink ? sink((size_t)total) : nullptr;
  if (!h) return POD_OK;   // sizes only
  std::fill(h, h + POD_HDR_WORDS, 0);
  h[0] = POD_IMAGE_MAGIC;
  h[1] = (int32_t)items.size();
  h[2] = G;
  h[3] = (int32_t)reqs.size();
  h[4] = n_groups;
  h[5] = (int32_t)reqs_off;
  h[6] = (int32_t)items_off;
  h[7] = (int32_t)groups_off;
  h[8] = (int32_t)counters_off;
  h[9] = n_slots;
  h[10] = kSlotFloats;
  h[11] = (int32_t)std::min<int64_t>(C, INT32_MAX);
  h[12] = (int32_t)wgs_off;
  h[13] = (int32_t)blocks_off;
  h[14] = (int32_t)n_blocks;
  h[15] = (int32_t)(items.size() - pool.size());
  h[16] = (int32_t)pool.size();
  h[17] = (int32_t)queue_off;
  h[18] = (int32_t)tdesc_off;
  for (size_t i = 0; i < reqs.size(); ++i) {
    int32_t* q = h + reqs_off + i * kReqWords;
    q[0] = reqs[i].qo_start;
    q[1] = reqs[i].qo_len;
    q[2] = reqs[i].kv_len;
    q[3] = reqs[i].page_start;
  }
  // Per-item row beside the item, read with it: a query tile's boundary data
  // (what an item boundary needs, without the request table); a key chunk's
  // request fields (so its loads need no request-table round trip).
  auto write_tdesc = [&](int32_t* td, const Item& it) {
    for (int x = 0; x < kTdescWords; ++x) td[x] = 0;
    const Req& q = reqs[it.w[1]];
    if (it.w[0] & kFlagChunk) {
      td[0] = q.qo_start;
      td[1] = q.qo_len;
      td[2] = q.kv_len;
      td[3] = q.page_start;
    } else {
      td[0] = q.qo_start + it.w[3];
      td[1] = it.w[4];
      td[2] = it.w[2];
      td[3] = q.kv_len - q.qo_len + it.w[3];
      td[4] = it.w[6];
      td[5] = q.kv_len;
    }
  };
  int n_pre = 0, n_dec = 0;
  int64_t k = 0, blk = 0;
  for (int w = 0; w < G; ++w) {
    const uint32_t* tl = listed.data() + bucket[(size_t)w * 3];
    const size_t nt = (size_t)(bucket[(size_t)w * 3 + 2] - bucket[(size_t)w * 3]);
    const uint32_t* cl = tl + nt;
    const size_t nc = (size_t)(bucket[(size_t)w * 3 + 3] - bucket[(size_t)w * 3 + 2]);
    int32_t* wg = h + wgs_off + (int64_t)w * kWgWords;
    bool chunks_first;
    if (nt == 0 || nc == 0) chunks_first = false;
    else if (d.order == POD_ORDER_PREFILL_FIRST) chunks_first = false;
    else if (d.order == POD_ORDER_DECODE_FIRST) chunks_first = true;
    else if (d.order == POD_ORDER_LONGEST_FIRST) {
      // the list holds each role's tiles heaviest first: compare with the
      // heavier of the two roles' first tiles
      int64_t tile_max = 0;
      for (size_t j = 0; j < nt; ++j) tile_max = std::max(tile_max, items[tl[j]].cost);
      chunks_first = items[cl[0]].cost > tile_max;
    }
    else chunks_first = ((w / kNumXcds) & 1) != 0;   // half of each die's workgroups each way
    wg[0] = (int32_t)k;
    wg[1] = (int32_t)nt;
    wg[2] = (int32_t)nc;
    wg[3] = (int32_t)blk;
    wg[5] = chunks_first ? 1 : 0;
    int64_t nb = 0;
    int32_t n_pre_tiles = 0, n_pre_blocks = 0;
    for (size_t j = 0; j < nt; ++j) {
      const Item& it = items[tl[j]];
      if ((it.w[0] & kFlagRole) == 0) {
        ++n_pre_tiles;
        n_pre_blocks += (it.w[6] - it.w[5] + kTileKeys - 1) / kTileKeys;
      }
      const int32_t lo = it.w[5], hi = it.w[6];
      const uint32_t meta = ((uint32_t)(it.w[0] & kFlagRole) << kEntRoleShift) |
                            ((uint32_t)it.w[2] << kEntKvhShift) | (uint32_t)j;
      for (int32_t kb = lo; kb < hi; kb += kTileKeys, ++nb) {
        int32_t* e = h + blocks_off + (blk + nb) * kBlockWords;
        e[0] = kb;
        e[1] = hi - 1;
        e[2] = reqs[it.w[1]].page_start;
        e[3] = (int32_t)(meta | (kb == lo ? kEntFirst : 0u));
      }
    }
    wg[4] = (int32_t)nb;
    wg[6] = n_pre_tiles;
    wg[7] = n_pre_blocks;
    blk += nb;
    for (size_t j = 0; j < nt + nc; ++j) {
      const Item& it = items[tl[j]];
      int32_t* dst = h + items_off + k * kItemWords;
      for (int x = 0; x < kItemWords; ++x) dst[x] = it.w[x];
      write_tdesc(h + tdesc_off + k * kTdescWords, it);
      ++k;
      ++((it.w[0] & kFlagRole) ? n_dec : n_pre);
    }
  }
  for (uint32_t i : pool) {
    const Item& it = items[i];
    int32_t* dst = h + items_off + k * kItemWords;
    for (int j = 0; j < kItemWords; ++j) dst[j] = it.w[j];
    write_tdesc(h + tdesc_off + k * kTdescWords, it);
    ++k;
    ++((it.w[0] & kFlagRole) ? n_dec : n_pre);
  }
  for (int i = 0; i < n_groups * kGroupWords; ++i) h[groups_off + i] = groups[i];
  for (int i = 0; i < n_groups; ++i) h[counters_off + i] = 0;
  h[queue_off] = 0;
  h[queue_off + 1] = 0;

  (void)n_pre;
  (void)n_dec;
  return POD_OK;
}

}  // namespace pod
