// Internal definitions shared by the host planner, the C ABI layer and the HIP
// kernels of the POD attention library. Host-only code includes this file too,
// so it names no HIP types.
#pragma once

#include <stdint.h>

#include <functional>
#include <string>

#include "pod_attn.h"

namespace pod {

constexpr int kHeadDim = 128;
constexpr int kThreads = 512;          // 8 wave64 per workgroup (2 per SIMD)
constexpr int kTileRows = 256;         // rows of a query-tile item (8 waves x 32)
constexpr int kTileKeys = 64;          // keys per block of a query tile
constexpr int kMaxGroup = 128;         // largest supported num_qo_heads / num_kv_heads
constexpr int kChunkRows = 32;         // max rows of a key-chunk item (one MFMA column block)
constexpr int kItemWords = 8;
constexpr int kReqWords = 4;
constexpr int kGroupWords = 4;
constexpr int kNumXcds = 8;            // MI355X: 8 accelerator dies, 32 CUs each
constexpr int kSlotFloats = kChunkRows * kHeadDim + kChunkRows;   // partial O + LSE
constexpr int kWgWords = 8;            // per-workgroup list header
constexpr int kBlockWords = 4;         // query-tile block-table entry
// Per-item row parallel to the items. A query tile's boundary data:
//   {first query row (qo_start + tok0), tokens, kv head, diagonal key of the
//    first token (kv_len - qo_len + tok0), key end of the item, kv_len, 0, 0};
// a key chunk's request fields: {qo_start, qo_len, kv_len, page_start, 0, 0, 0, 0}
constexpr int kTdescWords = 8;
constexpr int kMaxSinkHeads = 1024;    // sinks staged in LDS by the query tiles
constexpr int kMaxKvHeads = 16384;     // kv head index fits the block-table entry
constexpr int kMaxTilesPerWg = 65536;  // tile index fits the block-table entry
// Static scratch of the allocation-free entry point (one copy per device): the
// work-list image, then split-KV partial states.
constexpr size_t kStaticImageBytes = (size_t)16 << 20;
constexpr size_t kStaticPartialBytes = (size_t)48 << 20;
constexpr size_t kStaticScratchBytes = kStaticImageBytes + kStaticPartialBytes;
constexpr int kMaxDevices = 64;

// Block-table entry of a workgroup's query-tile stream:
//   {first key of the block, last key of its item, first page of the request, meta}
// meta: bit 31 first block of its item, bit 30 role, bits 16..29 kv head,
// bits 0..15 index of the item among the workgroup's query tiles.
// Header words of the work-list image (the layout pod_attn.h documents).
constexpr int kHdrReqs = 5, kHdrItems = 6, kHdrGroups = 7, kHdrCounters = 8, kHdrWgs = 12,
              kHdrBlocks = 13, kHdrPoolFirst = 15, kHdrPoolCount = 16, kHdrQueue = 17,
              kHdrTdesc = 18;

constexpr uint32_t kEntFirst = 1u << 31;
constexpr int kEntRoleShift = 30;
constexpr int kEntKvhShift = 16;

// item flags
constexpr int kFlagRole = 1;           // bit 0: 0 prefill, 1 decode
constexpr int kFlagChunk = 2;          // bit 1: key-chunk item
constexpr int kSplitShift = 8;

struct RoleParams {
  const void* q;
  int64_t q_st, q_sh;
  const void* k;
  const void* v;
  uint32_t kv_sp_b, kv_st_b, kv_sh_b;   // pool strides in bytes (< 2^31)
  const int32_t* indices;   // nullptr = identity page table
  void* out;
  int64_t o_st, o_sh;
  float* lse;               // nullptr = not requested
  float scale_log2;         // sm_scale * q_scale * k_scale * log2(e)
  float v_scale;            // output factor (the decode role's FP8 v_scale; else 1)
  int32_t causal;
  int32_t window_left;
  int32_t kv_fp8;           // K/V pools hold FP8 E4M3 (key-chunk items only)
};

struct Params {
  RoleParams role[2];
  // The work-list image in device memory. Everything a plan decides is read
  // from it (header words give the region offsets and the pool range), so the
  // launch arguments stay valid when a later plan rewrites the image in place:
  //   reqs, items, wgs (per workgroup: {first item, tiles, chunks, first block,
  //   blocks, chunks first, prefill tiles, prefill blocks}), blocks (query-tile
  //   block tables), tdesc (query-tile boundary rows), groups, counters and the
  //   queue {next pool item, workgroups done} (zero between launches); the
  //   shared key-chunk pool is items [pool_first, pool_first + pool_count).
  int32_t* image;
  float* partials;
  const float* sinks;       // nullptr = no sinks
  int32_t num_qo_heads;
  int32_t num_kv_heads;
  int32_t group_size;
  int32_t page_size;
  int32_t page_shift;       // log2(page_size) when it is a power of two, else -1
};

// Host planner (planner.cpp). It validates `d`, fills `info`, and asks `sink`
// for a buffer of info.image_ints words to write the work-list image into; a
// null sink, or a sink that returns nullptr, computes the sizes only.
// fixed_grid: launch d.num_cus workgroups whatever the plan holds (a captured
// launch keeps its grid across plans); otherwise a plan with fewer items than
// CUs gets one workgroup per item, rounded up to a multiple of the die count.
// The fixed grid's image is the larger one (the sizes to reserve).
using ImageSink = std::function<int32_t*(size_t)>;
int plan_compute(const pod_plan_desc& d, const ImageSink& sink, pod_plan_info& info,
                 std::string* err, bool fixed_grid);

// Launch the fused grid on `stream` (a hipStream_t); `done_event` (a hipEvent_t,
// or null) is signalled when the launch completes. Returns a hipError_t value.
int launch_pod_grid(const Params& p, int dtype, int grid, void* stream, void* done_event);
// Device address of the calling thread's current device's static scratch array
// (kStaticScratchBytes, 256-byte aligned), looked up once per device. `device`
// must be the current device. Returns a hipError_t value.
int static_scratch(int device, void** ptr);
// Cascade merge of n_pairs (row, head) states of head_dim 128 (merge_kernels.hip).
int launch_merge_states(const void* oa, const float* la, const void* ob, const float* lb,
                        void* oo, float* lo, int64_t n_pairs, int heads, int dtype,
                        const float* sinks, void* stream);

}  // namespace pod
