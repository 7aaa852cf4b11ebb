// Fused Prefill-On-Decode paged attention for gfx950 (MI355X, CDNA4).
//
// One launch of one persistent workgroup per CU runs the planner's work lists:
// query tiles (prefill style: up to 256 rows share each K/V block staged in
// LDS) and key chunks (decode style: the q_len x group rows of one request and
// kv head share every K/V row read from HBM; keys are split over the 8 waves
// and, for long requests, over workgroups).
// This is the "prefill and decode in one launch" idea of the POD article
// (www.dpshk.com/news/5405057, "POD 是什么"), built for wave64 and MFMA.
//
// Math per row (cuDNN backend article www.gsyq.cn/news/452757, "LSE 契约" and
// "Decode 能力矩阵与参数"): scores s_j = sm_scale * q.k_j over the row's valid
// keys, O = sum_j softmax_j v_j with an optional sink logit in the
// denominator, lse = log2 sum_j exp(s_j). The online softmax keeps the running
// max in raw score units and evaluates exp2(s * sm_scale * log2(e) - m'); partial
// states over disjoint key ranges merge as L = log2 sum 2^lse_k,
// O = sum 2^(lse_k - L) O_k.
//
// MFMA formulation (v_mfma_f32_32x32x16_{bf16,f16}):
//   S^T[key][row] = K[key][:] . Q[row][:]          A = K rows, B = Q^T (registers)
//   O^T[d][row]  += V^T[d][key] . P^T[key][row]    A = V^T, B = P^T (registers)
// The accumulators hold one query row per lane column, so the softmax row
// statistics are per-lane scalars plus one exchange between the lane halves
// (v_permlane32_swap). K rows are assigned to MFMA rows with bits 2 and 3 of
// the row index swapped, so each lane half's score accumulators cover 8
// consecutive keys and the P^T operand comes straight from them.
//
// LDS layout: one 256-byte row per key (one kv head's 128 dims). Key chunks
// (a block per wave, rows written from registers) permute the 16-byte chunks
// of row `key` by XOR with swz(key): sixteen consecutive keys then put any
// fixed chunk in 16 distinct bank groups (conflict-free row writes and K
// operand reads), and the 4-key x 16-dim blocks read by ds_read_b64_tr_b16 for
// the V^T operand fall in disjoint banks for the two 16-lane groups of each
// half wave. Query-tile ring slots keep the rows as the direct-to-LDS loads
// write them (four 256-byte rows per load instruction) and place row R at
// (R % 16) * group stride + (R / 16) * 256, with the group stride padded (1040
// bytes for K, 1088 for V) for the same bank spread.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <math.h>

#include <mutex>
#include <type_traits>

#include "pod_internal.h"

// Scratch memory of pod_run_static, for callers that cannot allocate: the
// work-list image followed by split-KV partial states. Every device the
// library runs on holds one copy until the process ends. Host code never uses
// this name as an address: it takes each device's copy from
// pod::static_scratch, which looks it up with hipGetSymbolAddress.
static __device__ __align__(256) char scratch[pod::kStaticScratchBytes];

namespace pod {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

template <typename T>
struct Dt;
template <>
struct Dt<__bf16> {
  using v8 = bf16x8;
  using v4 = bf16x4;
  static __device__ __forceinline__ f32x16 mfma(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16(v8 a, v8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <>
struct Dt<_Float16> {
  using v8 = f16x8;
  using v4 = f16x4;
  static __device__ __forceinline__ f32x16 mfma(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16(v8 a, v8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

constexpr int kRowBytes = kHeadDim * 2;       // one kv head's K row (16-bit types)
constexpr int kVRowBytes = kRowBytes + 64;    // V rows are padded by 64 bytes
constexpr int kStepKeys = 32;                 // keys per wave step of a key chunk
// Query-tile K block: row R sits in 1040-byte group R % 16 at slot R / 16, so
// each group is one lane-contiguous direct-to-LDS load of 4 rows, the 16
// rows read at one 16-byte chunk fall in 16 distinct bank groups, and the
// chunk offset of a fragment read is an instruction constant.
constexpr int kTileKGroup = 4 * kRowBytes + 16;
constexpr int kTileKBytes = 16 * kTileKGroup;                               // 16.25 KB
// Query-tile V block: row R sits in 1088-byte group R % 16 at slot R / 16, so
// the 4 consecutive rows of a transpose read land 16 banks apart.
constexpr int kTileVGroup = 4 * kRowBytes + 64;
constexpr int kTileBuf = kTileKBytes + 16 * kTileVGroup;                    // 33.25 KB per buffer
constexpr int kWaveKBytes = kStepKeys * kRowBytes;
constexpr int kWaveLds = kWaveKBytes + kStepKeys * kVRowBytes;              // 18 KB
constexpr int kWaves = kThreads / 64;                                      // 8 waves
constexpr int kRingSlots = 4;                                               // query-tile ring
constexpr int kIdSlot = kWaves * 256;                                       // page ids, one ring slot
// merge of the key-chunk waves: maxima and sums of 8 waves, 4 partial O sums
constexpr int kMergeLds = (2 * kWaves * 32 + 4 * kHeadDim * 32) * 4 + 16;
constexpr int kMax2(int a, int b) { return a > b ? a : b; }
// one LDS array: the query tile's ring slots, or one 18 KB part per key-chunk wave
constexpr int kLdsMain = kMax2(kMax2(kRingSlots * kTileBuf, kWaves * kWaveLds), kMergeLds);
static_assert(kLdsMain + kRingSlots * kIdSlot <= 160 * 1024, "LDS budget");
// the running max moves only when a block's max exceeds it by this much (log2 units)
constexpr float kRescaleThreshold = 8.f;
// Query tiles: largest sum of one block's exponentials (one lane, 32 keys) taken
// without moving the row's reference maximum.
constexpr float kBlockSumLimit = 0x1p64f;
// Start of a query-tile row's running max (raw score units): finite, so the
// bound test and the exponent need no case for a row that has seen no valid
// key yet. The max is only a reference point (P = exp2(sl2 (s - m)) for any m
// that keeps sl2 (s - m) below the threshold): the first block with a valid key
// usually moves it, scaling the still-zero state by exp2(-huge) = 0, and while
// no key is valid every exponent is -inf.
constexpr float kMaxInit = -1e30f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Maximum of two or three scores with one instruction and no NaN quieting
// (scores are finite or -inf; fmaxf adds a canonicalising max per operand).
__device__ __forceinline__ float max3_raw(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float max_raw(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Value from the other lane half (lane ^ 32) combined with the own value.
__device__ __forceinline__ float xhalf_max(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// MFMA row m of a 32-key score block holds key key_row(m) of that block.
__device__ __forceinline__ int key_row(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}
// key (within a 32-key block) held by score accumulator j of lane half hi
__device__ __forceinline__ int acc_key(int j, int hi) { return 16 * (j >> 3) + 8 * hi + (j & 7); }
// head-dim index (within a 32-wide block) held by output accumulator j of lane half hi
__device__ __forceinline__ int acc_d(int j, int hi) { return 8 * (j >> 2) + 4 * hi + (j & 3); }

// K blocks: 16-byte chunk c of row `key` is stored at slot c ^ swz(key)
// (depends on key % 16 only), so 16 consecutive rows read at one chunk hit
// 16 distinct bank groups.
__device__ __forceinline__ int swz(int key) { return ((key & 3) << 2) | ((key >> 2) & 3); }

// The query tile's direct-to-LDS ring is managed by hand: its loads are
// issued through inline asm, so the compiler neither tracks them nor adds
// waits of its own (compiler-tracked loads lose track of which LDS slot each
// one targets across the loop back edge and then drain every outstanding
// load), and the ring waits with explicit vmcnt counts.
//
// One 16-byte (dwordx4) or 4-byte (dword) load per lane from global `src`
// into LDS at the wave-uniform address `dst` + 16 (or 4) x lane.
__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const LDS_AS char*)p);
}
__device__ __forceinline__ void lds_dma16(const void* src, const char* dst) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(src), "s"(lds_addr(dst)) : "memory", "m0");
}
// the same with the LDS destination given as a wave-uniform LDS byte address
__device__ __forceinline__ void lds_dma16_at(const void* src, uint32_t dst) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(src), "s"(dst) : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4_at(const void* src, uint32_t dst) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :: "v"(src), "s"(dst) : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4(const void* src, const char* dst) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :: "v"(src), "s"(lds_addr(dst)) : "memory", "m0");
}
// Wait until at most N vector-memory loads of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}
// Workgroup barrier without a fence: each wave has already waited for its
// own ring loads (a fence would wait for every outstanding load, including
// the blocks still streaming in).
__device__ __forceinline__ void ring_barrier() { asm volatile("s_barrier" ::: "memory"); }

template <typename T>
__device__ __forceinline__ u32x4 ld16(const T* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x4 lds_ld16(const char* base, int off) {
  return *reinterpret_cast<const u32x4*>(base + off);
}
__device__ __forceinline__ void lds_st16(char* base, int off, u32x4 v) {
  *reinterpret_cast<u32x4*>(base + off) = v;
}

// V^T operand of one 32x32x16 MFMA from a padded row-major V block: lane
// (d = l % 32, half hi = l / 32) gets V[key0 + 8*hi + e][d0 + l % 32], e = 0..7.
// Each ds_read_b64_tr_b16 serves 4 keys x 16 dims per 16-lane group; `vlane`
// is the lane's constant part of the address (see vt_lane), the rest folds into
// the instruction offset.
template <typename V8>
__device__ __forceinline__ V8 vt_operand(const char* vlane, int key0, int d0) {
  u32x2 part[2];
#pragma unroll
  for (int ld = 0; ld < 2; ++ld) {
    const LDS_AS char* p = (const LDS_AS char*)vlane + (key0 + 4 * ld) * kVRowBytes + d0 * 2;
    i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)p);
    part[ld] = __builtin_bit_cast(u32x2, v);
  }
  u32x4 w = {part[0][0], part[0][1], part[1][0], part[1][1]};
  return __builtin_bit_cast(V8, w);
}
// lane-dependent byte offset for vt_operand: row 8*(g/2) + i/4, dims 16*(g%2) + 4*(i%4)
__device__ __forceinline__ int vt_lane(int lane) {
  const int g = lane >> 4, i = lane & 15;
  return (8 * (g >> 1) + (i >> 2)) * kVRowBytes + (16 * (g & 1) + 4 * (i & 3)) * 2;
}

struct RowGeom {
  int qo_start, qo_len, kv_len, page_start;
};

struct RoleView {
  const void* q;
  int64_t q_st, q_sh;
  const char* k;            // pool base + this item's kv head offset
  const char* v;
  uint32_t kv_sp_b, kv_st_b;
  const int32_t* indices;
  void* out;
  int64_t o_st, o_sh;
  float* lse;
  float scale_log2;
  float v_scale;            // output factor (FP8 calibration; 1 otherwise)
  int causal, window_left;
};

// Kernel parameters are read in place from the kernarg segment (through the
// scalar unit) where they are used, rather than all loaded at entry and held
// in scalar registers for the whole launch.
using PArg = const __attribute__((address_space(4))) Params&;
// the same reference, opaque to the compiler: loads through it stay where they
// are written (not hoisted out of the loop that contains them)
__device__ __forceinline__ PArg reload(PArg p) {
  const __attribute__((address_space(4))) Params* q = &p;
  asm volatile("" : "+s"(q));
  return *q;
}

__device__ __forceinline__ RoleView pick_role(PArg p, int role, int kvh) {
  const __attribute__((address_space(4))) RoleParams& a = p.role[0];
  const __attribute__((address_space(4))) RoleParams& b = p.role[1];
  RoleView r;
  r.q = role ? b.q : a.q;
  r.q_st = role ? b.q_st : a.q_st;
  r.q_sh = role ? b.q_sh : a.q_sh;
  const uint32_t sh = role ? b.kv_sh_b : a.kv_sh_b;
  r.k = reinterpret_cast<const char*>(role ? b.k : a.k) + (uint64_t)kvh * sh;
  r.v = reinterpret_cast<const char*>(role ? b.v : a.v) + (uint64_t)kvh * sh;
  r.kv_sp_b = role ? b.kv_sp_b : a.kv_sp_b;
  r.kv_st_b = role ? b.kv_st_b : a.kv_st_b;
  r.indices = role ? b.indices : a.indices;
  r.out = role ? b.out : a.out;
  r.o_st = role ? b.o_st : a.o_st;
  r.o_sh = role ? b.o_sh : a.o_sh;
  r.lse = role ? b.lse : a.lse;
  r.scale_log2 = role ? b.scale_log2 : a.scale_log2;
  r.v_scale = role ? b.v_scale : a.v_scale;
  r.causal = role ? b.causal : a.causal;
  r.window_left = role ? b.window_left : a.window_left;
  return r;
}

// Physical page of logical key `key` and the byte offset of its row in the pool.
__device__ __forceinline__ uint32_t page_of(const RoleView& r, PArg p, int page_start, int key) {
  const int pg = p.page_shift >= 0 ? (key >> p.page_shift) : key / p.page_size;
  return r.indices ? (uint32_t)r.indices[page_start + pg] : (uint32_t)(page_start + pg);
}
__device__ __forceinline__ uint64_t row_off(const RoleView& r, PArg p, uint32_t page, int key) {
  const int slot = p.page_shift >= 0 ? (key & (p.page_size - 1)) : key % p.page_size;
  return (uint64_t)page * r.kv_sp_b + (uint32_t)slot * r.kv_st_b;
}

// Where one wave's key rows of a key chunk come from: pool bases of the item's
// kv head, page table and strides, the wave's first key, the chunk's last key.
struct KeySrc {
  const char* k;
  const char* v;
  const int32_t* indices;
  uint32_t sp_b, st_b;
  int page_start, first, last;
};

// The loads a 16-bit key chunk keeps in flight at the top of its step loop:
// the rows of the current step and the page ids of the one after. A chunk
// issues them for the next chunk of the workgroup's list while it merges its
// waves and stores its output, so the load stream does not stop there.
struct ChunkCarry {
  uint32_t pidx[8];
  u32x4 kst[8], vst[8];
};

// Q^T operand of one row: lane half hi holds d = hi*64 + c*8 + [0,8) for MFMA c.
template <typename T>
__device__ __forceinline__ void load_q(typename Dt<T>::v8 (&qreg)[8], const RoleView& r,
                                       bool ok, int tok_global, int head, int hi) {
  const T* qp = reinterpret_cast<const T*>(r.q) + (int64_t)tok_global * r.q_st +
                (int64_t)head * r.q_sh + hi * 64;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    u32x4 x = ok ? ld16(qp + c * 8) : u32x4{0, 0, 0, 0};
    qreg[c] = __builtin_bit_cast(typename Dt<T>::v8, x);
  }
}

// Row range of the mask in "offset, span" form: key k is valid iff
// (unsigned)(k - lo) <= span. Empty ranges never match.
struct RowMask {
  int lo;
  unsigned span;
};
__device__ __forceinline__ RowMask row_mask(int key_lo, int key_hi) {
  RowMask m;
  if (key_hi < key_lo) {
    m.lo = 1 << 30;
    m.span = 0;
  } else {
    m.lo = key_lo;
    m.span = (unsigned)(key_hi - key_lo);
  }
  return m;
}

// Running-max update for NB score blocks of one lane (raw scores, masked
// entries already -inf). m is kept in raw units and only moves when a block max
// exceeds it by kRescaleThreshold (log2 units), so P stays below 2^threshold
// and O and l are rescaled rarely.
template <int NB>
__device__ __forceinline__ void update_max(f32x16 (&s)[NB], float sl2, float& m, float& l,
                                           f32x16 (&o)[4]) {
  float mx0 = kNegInf, mx1 = kNegInf;
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int j = 0; j < 16; j += 2) {
      mx0 = fmaxf(mx0, s[b][j]);
      mx1 = fmaxf(mx1, s[b][j + 1]);
    }
  float mx = xhalf_max(fmaxf(mx0, mx1));
  const bool upd = (m == kNegInf) ? (mx != kNegInf) : ((mx - m) * sl2 > kRescaleThreshold);
  if (__any(upd)) {
    const float mn = upd ? mx : m;
    const float alpha = upd ? fast_exp2((m - mn) * sl2) : 1.f;
    l *= alpha;
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int j = 0; j < 16; ++j) o[b][j] *= alpha;
    m = mn;
  }
}

// P = exp2(s * sl2 - mu2) of one 32-key score block as two MFMA operands.
template <typename T>
__device__ __forceinline__ void exp_block(const f32x16& s, float sl2, float mu2, float& l,
                                          typename Dt<T>::v8 (&pb)[2]) {
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float e = fast_exp2(fmaf(s[8 * h + i], sl2, -mu2));
      l += e;
      pb[h][i] = (T)e;
    }
}

template <typename T, int NB>
__device__ __forceinline__ void softmax_step(f32x16 (&s)[NB], float sl2, float& m, float& l,
                                             f32x16 (&o)[4], typename Dt<T>::v8 (&pb)[NB][2]) {
  update_max<NB>(s, sl2, m, l, o);
  const float mu2 = (m == kNegInf) ? 0.f : m * sl2;
#pragma unroll
  for (int b = 0; b < NB; ++b) exp_block<T>(s[b], sl2, mu2, l, pb[b]);
}

// ----------------------------------------------------------------------------
// Query tiles: up to 256 rows (tokens x group heads) of one request and kv head
// over the item's keys in 64-key blocks; wave w owns rows 32w + [0, 32). A
// workgroup runs all of its query tiles as one stream of blocks (the planner's
// block table): K/V blocks go straight from HBM/L2 to LDS (16-byte direct
// loads) through a ring of 4 slots, two blocks ahead of the one computed, so
// the next tile's page ids and first blocks are in flight while the current
// tile finishes. The eight waves share every block (two per SIMD, so one
// wave's exponentials run beside the other's MFMAs).
template <bool kPow2>
struct PageMap {
  int shift, mask, size;
  __device__ __forceinline__ int page(int key) const { return kPow2 ? key >> shift : key / size; }
  __device__ __forceinline__ int slot(int key) const { return kPow2 ? key & mask : key % size; }
};

// Read-only plan words through the scalar unit (the plan is constant during
// a launch).
using CI32 = const __attribute__((address_space(4))) int32_t;
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
using CI32x4 = const __attribute__((address_space(4))) i32x4;
__device__ __forceinline__ CI32* plan_words(const int32_t* p) { return (CI32*)p; }
// header word i of the work-list image (uniform: one scalar load)
__device__ __forceinline__ int hdr_word(PArg p, int i) { return plan_words(p.image)[i]; }
// image region whose offset is header word i
__device__ __forceinline__ int32_t* image_region(PArg p, int i) { return p.image + hdr_word(p, i); }

// one query-tile item, wave-uniform (its boundary row of the plan: one
// 32-byte scalar load)
struct TileDesc {
  int qrow0, ntok, kvh, diag0, kv_end, kv_len;
};
__device__ __forceinline__ TileDesc tile_desc(CI32* tdesc, int idx) {
  typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
  const i32x8 w = *reinterpret_cast<const __attribute__((address_space(4))) i32x8*>(tdesc + idx * kTdescWords);
  return TileDesc{w[0], w[1], w[2], w[3], w[4], w[5]};
}


template <typename T, bool kPow2, int kPaged>
__device__ __forceinline__ void tile_stream(PArg p, int role, const int32_t* ttd, int t0, int nt, const int32_t* tab,
                            int nv, char* ring, char* idring, float* sink_lds, char* pf_lds) {
  using V8 = typename Dt<T>::v8;
  CI32* ctab = plan_words(tab);
  CI32* ctd = plan_words(ttd);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r32 = lane & 31, hi = lane >> 5;
  const int g = p.group_size;
  const int row = wave * 32 + r32;
  const bool second = wave >= kWaves / 2;   // wave-uniform: the V-first half
  const PageMap<kPow2> pm{p.page_shift, p.page_size - 1, p.page_size};
  // the role's K/V pools (kv head 0), page table and strides: all the block
  // loads need; the rest of the role is read again at item boundaries
  const RoleView r = pick_role(p, role, 0);
  const char* const kpool = r.k;
  const char* const vpool = r.v;
  // kPaged: 1 the role has a page table, 0 identity pages, 2 read here (the
  // power-of-two page sizes, which every serving workload uses, get the first
  // two as separate code: no select between the two page sources per load)
  const bool paged = kPaged == 2 ? r.indices != nullptr : kPaged == 1;
  // page-id loads read the page table, or word 0 of the request table (unused)
  const int32_t* const id_src = paged ? r.indices : image_region(p, kHdrReqs);
  const uint32_t kv_sp = r.kv_sp_b, kv_st = r.kv_st_b;
  const uint32_t kv_sh = role ? p.role[1].kv_sh_b : p.role[0].kv_sh_b;

  // block v's entry (blocks past the end repeat the last one), one 16-byte
  // scalar load; each pass loads the entries it needs at its start and carries
  // those of the blocks it computes from earlier passes
  struct Ent {
    int kb, kl, ps;
    uint32_t meta;
  };
  auto ent = [&](int v) {
    const i32x4 e = reinterpret_cast<CI32x4*>(ctab)[min(v, nv - 1)];
    return Ent{e[0], e[1], e[2], (uint32_t)e[3]};
  };
  auto is_first = [](const Ent& e) { return (e.meta & kEntFirst) != 0; };
  auto item_idx = [](const Ent& e) { return (int)(e.meta & 0xffff); };

  // Direct loads: wave w fills groups 2w+u (u = 0, 1) of K and of V; group i
  // holds rows i + 16 (lane / 16), lane & 15 is the 16-byte slot. K row R sits at
  // (R % 16) * 1040 + (R / 16) * 256, V row R at (R % 16) * 1088 + (R / 16) * 256.
  // Rows past the item's last key repeat that key (finite values the mask sends
  // to -inf), and blocks past the end of the stream load the last block again,
  // so every iteration issues the same loads.
  const int lq = lane >> 4, lslot = lane & 15;
  int rr[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) rr[u] = 2 * wave + u + 16 * lq;
  // Page ids stream through a per-wave LDS ring too (lane l holds the page of
  // key kb + l); without a page table the loads read word 0 of the request
  // table and the identity page is used instead.
  auto idslot = [&](int v) { return idring + (v & (kRingSlots - 1)) * kIdSlot + wave * 256; };
  auto slot = [&](int v) { return ring + (v & (kRingSlots - 1)) * kTileBuf; };
  // the same slots as LDS byte addresses (wave-uniform), for the direct loads
  const uint32_t ring_at = lds_addr(ring), idring_at = lds_addr(idring) + wave * 256;
  auto load_ids = [&](int v, const Ent& e) {
    const int kb = e.kb, kl = e.kl, ps = e.ps;
    const uint32_t pl = (uint32_t)pm.page(min(kb + lane, kl));
    lds_dma4_at(id_src + (paged ? ps + pl : 0u), idring_at + (v & (kRingSlots - 1)) * kIdSlot);
  };
  int32_t pid[2];
  auto read_ids = [&](int v) {
#pragma unroll
    for (int u = 0; u < 2; ++u) pid[u] = *reinterpret_cast<const int32_t*>(idslot(v) + rr[u] * 4);
  };
  // the K and V loads of the wave's row group u of block v
  auto dma_rows = [&](int v, int u, const Ent& e) {
    const int kb = e.kb, kl = e.kl, ps = e.ps;
    // the block's kv head: a wave-uniform offset of both pools
    const uint64_t hoff = (uint64_t)((e.meta >> kEntKvhShift) & 0x3fff) * kv_sh;
    const int key = min(kb + rr[u], kl);
    const uint32_t page = paged ? (uint32_t)pid[u] : (uint32_t)(ps + pm.page(key));
    const uint64_t ro = (uint64_t)page * kv_sp + ((uint32_t)pm.slot(key) * kv_st + (lslot << 4));
    const uint32_t dst = ring_at + (v & (kRingSlots - 1)) * kTileBuf;
    lds_dma16_at(kpool + hoff + ro, dst + (2 * wave + u) * kTileKGroup);
    lds_dma16_at(vpool + hoff + ro, dst + kTileKBytes + (2 * wave + u) * kTileVGroup);
  };
  auto dma_block = [&](int v, const Ent& e) {
    dma_rows(v, 0, e);
    dma_rows(v, 1, e);
  };

  // K operand: lane reads row h*32 + key_row(r32), chunk hi*8 + c, at
  // klane + h*512 + c*16
  const int krow = key_row(r32);
  const int klane = (krow & 15) * kTileKGroup + (krow >> 4) * kRowBytes + hi * 128;
  // V^T operand: lane rows 8(g/2) + i/4, dims 16(g%2) + 4(i%4)
  const int vg = lane >> 4, vi = lane & 15;
  const int vlane = kTileKBytes + (8 * (vg >> 1) + (vi >> 2)) * kTileVGroup +
                    (16 * (vg & 1) + 4 * (vi & 3)) * 2;

  // entries of the blocks computed next (block t and t + 1 of a pass)
  Ent ea = ent(0), eb = ent(1);
  // the item whose softmax state (rm, m, l, o) is live
  int cur = item_idx(ea);
  V8 qreg[8];
  f32x16 o[4];
  // running max (raw units) and row sum (this lane half's keys)
  float m = kMaxInit, l = 0.f, sl2 = 0.f;
  RowMask rm;
  // this lane's row of item d: token, qo head; false past the item's rows
  // the lane's token offset and group head within any tile
  const int rdiv = row / g, rmod = row % g;
  // this lane's row of item d: token offset in the tile, qo head; false past
  // the item's rows
  auto geom = [&](const TileDesc& d, int& toff, int& head) {
    const bool ok = row < d.ntok * g;
    toff = ok ? rdiv : 0;
    head = d.kvh * g + (ok ? rmod : 0);
    return ok;
  };
  // item i of the list, and its role, read again where they are needed
  // a use of the query registers: the compiler waits here for the query loads
  // (vmcnt(0), with every load issued before them), so no wait for them is
  // left in the loop.
  // The next item's query: load c' brings 32 contiguous bytes of each row (16
  // per lane half: d = 16 c' + 8 hi + [0, 8)), then one swap between the lane
  // halves per register gives the MFMA layout (lane half hi holds d = 64 hi +
  // 8 c + [0, 8) in qreg[c]). Using the loaded values makes the compiler wait
  // for them there (vmcnt(0), with every load issued before them), so no wait
  // for the query is left in the loop.
  u32x4 qraw[8];
  auto load_query = [&](int i) {
    PArg q = reload(p);
    const TileDesc d = tile_desc(ctd, i);
    int toff, head;
    const bool ok = geom(d, toff, head);
    const RoleView r = pick_role(q, role, 0);
    const T* qp = reinterpret_cast<const T*>(r.q) + (int64_t)(d.qrow0 + toff) * r.q_st +
                  (int64_t)head * r.q_sh + hi * 8;
#pragma unroll
    for (int c = 0; c < 8; ++c) qraw[c] = ok ? ld16(qp + c * 16) : u32x4{0, 0, 0, 0};
  };
  auto query_landed = [&]() {
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // lower half keeps qraw[c] and takes the upper half's; the upper half
        // gets the lower half's qraw[c + 4] and keeps its own
        const auto sw = __builtin_amdgcn_permlane32_swap(qraw[c][w], qraw[c + 4][w], false, false);
        qraw[c][w] = sw[0];
        qraw[c + 4][w] = sw[1];
      }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      qreg[2 * c] = __builtin_bit_cast(V8, qraw[c]);
      qreg[2 * c + 1] = __builtin_bit_cast(V8, qraw[c + 4]);
    }
  };
  auto setup = [&](int i) {
    PArg q = reload(p);
    const TileDesc d = tile_desc(ctd, i);
    const RoleView r = pick_role(q, role, 0);
    int toff, head;
    geom(d, toff, head);
    const int pdiag = d.diag0 + toff;
    const int key_hi = min(r.causal ? pdiag : d.kv_len - 1, d.kv_end - 1);
    const int key_lo = r.window_left >= 0 ? max(0, pdiag - r.window_left) : 0;
    rm = row_mask(key_lo, key_hi);
    sl2 = r.scale_log2;
    m = kMaxInit;
    l = 0.f;
#pragma unroll
    for (int b = 0; b < 4; ++b) o[b] = f32x16{};
  };
  // normalise (sink folded into the denominator) and store O and the LSE of item d
  auto finish = [&](int i) {
    PArg q = reload(p);
    const TileDesc d = tile_desc(ctd, i);
    const RoleView r = pick_role(q, role, 0);
    int toff, head;
    const bool ok = geom(d, toff, head);
    const float lt = xhalf_sum(l);
    // log2 offset of the row's values (if no key was valid, l is 0 and a sink
    // term comes out +inf, so O = 0)
    const float mu2 = m * sl2;
    float den = lt;
    if (q.sinks) den += fast_exp2(sink_lds[head] * kLog2e - mu2);
    const float inv = den > 0.f ? r.v_scale / den : 0.f;
    // Output accumulator j = 4a + c of lane half hi is d = db*32 + 8a + 4hi + c.
    // Per pair a = 2b, 2b+1 one swap between the lane halves (all lanes take
    // part) leaves each half 8 consecutive d: the lower half d = 16b + [0, 8),
    // the upper d = 16b + 8 + [0, 8), so each store writes 32 contiguous bytes
    // of a row.
    u32x4 ow[4][2];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        typename Dt<T>::v4 pw, qw;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          pw[c] = (T)(o[db][8 * b + c] * inv);
          qw[c] = (T)(o[db][8 * b + 4 + c] * inv);
        }
        u32x2 P = __builtin_bit_cast(u32x2, pw), Q = __builtin_bit_cast(u32x2, qw);
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          const auto sw = __builtin_amdgcn_permlane32_swap(P[w], Q[w], false, false);
          P[w] = sw[0];
          Q[w] = sw[1];
        }
        ow[db][b] = u32x4{P[0], P[1], Q[0], Q[1]};
      }
    // outputs are written once and not read again in the launch: non-temporal
    // stores stream them out now instead of leaving dirty lines in L2 for the
    // write-back at the end of the launch
    if (ok) {
      T* op = reinterpret_cast<T*>(r.out) + (int64_t)(d.qrow0 + toff) * r.o_st + (int64_t)head * r.o_sh + hi * 8;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int b = 0; b < 2; ++b) __builtin_nontemporal_store(ow[db][b], reinterpret_cast<u32x4*>(op + db * 32 + 16 * b));
      if (r.lse && hi == 0)
        __builtin_nontemporal_store(lt > 0.f ? mu2 + fast_log2(lt) : kNegInf, &r.lse[(int64_t)(d.qrow0 + toff) * q.num_qo_heads + head]);
    }
  };

  // Each block b is two phases of a wave:
  //   M: the score MFMAs of block b (S_b, 16, K from LDS slot b) and the P.V
  //      MFMAs of block b-1 (16, V^T from slot b-1, P_{b-1} in registers);
  //   V: mask and exponentials of S_b (P_b and l), VALU only; the running
  //      max moves only when a block's sum shows it must.
  // Waves 0-3 run M while waves 4-7 (the other wave of each SIMD) run V, then
  // the other way round, with a barrier between the turns: the MFMA pipe takes
  // one wave's 32 MFMAs while the VALU runs the other wave's softmax.
  f32x16 s[2];
  s[0] = f32x16{};
  s[1] = f32x16{};
  V8 pb[2][2];
  auto m_s = [&](int b) {
    const char* kb_buf = slot(b);
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const u32x4 kf = lds_ld16(kb_buf + klane, 2 * h * kRowBytes + c * 16);
        s[h] = Dt<T>::mfma(__builtin_bit_cast(V8, kf), qreg[c], s[h]);
      }
  };
  auto m_pv = [&](int b) {
    const char* vb = slot(b) + vlane;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int mp = 0; mp < 2; ++mp)
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          // rows 32 h + 16 mp + [lane part] + 4 ld: slot-row 2 h + mp of the groups
          u32x2 part[2];
#pragma unroll
          for (int ld = 0; ld < 2; ++ld) {
            const LDS_AS char* pp = (const LDS_AS char*)vb + 4 * ld * kTileVGroup +
                                    (2 * h + mp) * kRowBytes + db * 64;
            part[ld] = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)pp));
          }
          const u32x4 w = {part[0][0], part[0][1], part[1][0], part[1][1]};
          o[db] = Dt<T>::mfma(__builtin_bit_cast(V8, w), pb[h][mp], o[db]);
        }
  };
  // M with both parts: score and P.V MFMAs alternate, LDS reads ahead of them.
  auto m_both = [&](int b) {
    m_s(b);
    m_pv(b - 1);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
    }
  };
  auto v_phase = [&](int kb) {
    if (__any((unsigned)(kb - rm.lo) > rm.span || (unsigned)(kb + kTileKeys - 1 - rm.lo) > rm.span)) {
      // key of accumulator j = kb + 8 hi + (its constant part); the lane part
      // is opaque so that the 32 key offsets are not held in registers
      int base = 8 * hi;
      asm volatile("" : "+v"(base));
      base += kb - rm.lo;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int kidx = base + h * 32 + acc_key(j, 0);
          s[h][j] = ((unsigned)kidx <= rm.span) ? s[h][j] : kNegInf;
        }
    }
    // Exponentials against the row's current reference m (raw units, the
    // same in both lane halves of a row), then one test of the block's sum:
    // it passes 2^64 only if a score sits far above m (always in a row's
    // first block with a valid key, whose m is still kMaxInit; rarely after),
    // and only then is the block maximum taken, the state rescaled and the
    // exponentials redone. Below that bound P, l and O stay finite in fp32
    // and bf16, and their ratio does not depend on m.
    float la[4];
    auto exps = [&](float mu2) __attribute__((always_inline)) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float e = fast_exp2(fmaf(s[h][8 * hh + i], sl2, -mu2));
            la[i & 3] = (h == 0 && hh == 0 && i < 4) ? e : la[i & 3] + e;
            pb[h][hh][i] = (T)e;
          }
    };
    // (kMaxInit * sl2 is finite for every accepted scale; while no key is
    // valid every score is -inf and every exponential 0)
    exps(m * sl2);
    float bsum = (la[0] + la[1]) + (la[2] + la[3]);
    if (__any(!(bsum <= kBlockSumLimit))) {
      // block max: two chains of three-way maxima, then the other lane half
      float mx0 = max3_raw(s[0][0], s[0][1], s[0][2]);
      float mx1 = max3_raw(s[1][0], s[1][1], s[1][2]);
#pragma unroll
      for (int j = 3; j < 15; j += 2) {
        mx0 = max3_raw(mx0, s[0][j], s[0][j + 1]);
        mx1 = max3_raw(mx1, s[1][j], s[1][j + 1]);
      }
      mx0 = max3_raw(mx0, s[0][15], s[1][15]);
      {
        const float mx = max3_raw(mx0, mx1, m);
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx0 = max_raw(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      }
      // the reference only moves up; rows whose block stays below it keep it
      // and scale by exp2(0) = 1
      const float alpha = fast_exp2((m - mx0) * sl2);
      l *= alpha;
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int j = 0; j < 16; ++j) o[b][j] *= alpha;
      m = mx0;
      exps(m * sl2);
      bsum = (la[0] + la[1]) + (la[2] + la[3]);
    }
    l += bsum;
  };

  // Block v streams into ring slot v % 4 and its page ids into id slot v % 4.
  // Iteration t reads slots t-1 and t and issues the K/V loads of block t+2
  // (4 loads, into the slot of block t-2) and then the ids of block t+6 (1
  // load), and moves the ids of block t+3 to registers. Waves 0-3 issue all of
  // it at the start of their softmax turn, so their MFMA turn holds no load
  // work (a wave that mixes other instructions into its MFMA stream issues the
  // MFMAs more slowly); waves 4-7 issue theirs around their MFMA turn, which
  // keeps their loads a turn further ahead. The prologue issues what
  // iterations -2 and -1 would have, after the sinks (LDS copy, for the tiles'
  // final normalisation) and the first tile's query.
  setup(cur);
  load_query(cur);
  // Pull the block table and the tiles' boundary rows into L2 (one word per
  // 64-byte line, up to 16 KB each), so the scalar loads of them hit there;
  // the words land in a scratch LDS area nobody reads.
  {
    const int lines = min((nv * kBlockWords * 4 + 63) / 64, 256);
    for (int c = wave; c * 64 < lines; c += kWaves)
      lds_dma4(tab + min(c * 64 + lane, lines - 1) * 16, pf_lds);
    const int tlines = min((nt * kTdescWords * 4 + 63) / 64, 256);
    for (int c = wave; c * 64 < tlines; c += kWaves)
      lds_dma4(ttd + t0 * kTdescWords + min(c * 64 + lane, tlines - 1) * 16, pf_lds);
  }
  if (p.sinks) {
    for (int c = wave; c * 64 < p.num_qo_heads; c += kWaves)
      lds_dma4(p.sinks + min(c * 64 + lane, p.num_qo_heads - 1), (char*)sink_lds + c * 256);
  }
  load_ids(0, ea);
  load_ids(1, eb);
  load_ids(2, ent(2));
  load_ids(3, ent(3));
  wait_vm<3>();
  read_ids(0);
  dma_block(0, ea);
  load_ids(4, ent(4));
  wait_vm<7>();
  read_ids(1);
  dma_block(1, eb);
  load_ids(5, ent(5));
  wait_vm<11>();
  read_ids(2);
  query_landed();

  // iteration t: wait for block t, then issue block t+2's loads
  auto top = [&](int t) {
    // block t landed (and the ids of block t+3, issued before it); the 6 loads
    // issued after it may still be in flight
    wait_vm<6>();
    ring_barrier();
  };
  // Item boundaries: block t opens a new item (first block): after the M turn
  // that ends the previous item's P.V, that item is normalised and stored and
  // the new one's state reset (the stores follow the loads of block t+2 and
  // make the wait for that block count them too, which only delays it until
  // they have drained). Block t closes its item (the next
  // block opens one): after the M turn of S_t the next item's query goes to the
  // registers and is waited for at once (with every load issued before it):
  // one load latency per item, and no wait on the query in the other passes.
  if (!second) {
    // waves 0-3, iteration t: M(t), barrier, V(t)
    // e2, e6: entries of blocks t+2 and t+6, loaded one pass ahead
    Ent e2 = ent(2), e6 = ent(6);
    {
      top(0);
      m_s(0);
      ring_barrier();
      dma_rows(2, 0, e2);
      dma_rows(2, 1, e2);
      load_ids(6, e6);
      read_ids(3);
      if (nv > 1 && is_first(eb)) {
        load_query(item_idx(eb));
        query_landed();
      }
      const Ent n2 = ent(3), n6 = ent(7);
      v_phase(ea.kb);
      ea = eb;
      eb = e2;
      e2 = n2;
      e6 = n6;
    }
    for (int t = 1; t < nv; ++t) {
      const bool bnd = is_first(ea);
      const bool nq = t + 1 < nv && is_first(eb);
      top(t);
      m_both(t);
      ring_barrier();
      dma_rows(t + 2, 0, e2);
      dma_rows(t + 2, 1, e2);
      load_ids(t + 6, e6);
      read_ids(t + 3);
      if (bnd) {
        finish(cur);
        cur = item_idx(ea);
        setup(cur);
      }
      if (nq) {
        load_query(item_idx(eb));
        query_landed();
      }
      // next pass's entries: issued where no LDS wait follows until the next
      // pass (scalar and LDS loads share one counter)
      const Ent n2 = ent(t + 3), n6 = ent(t + 7);
      v_phase(ea.kb);
      ea = eb;
      eb = e2;
      e2 = n2;
      e6 = n6;
    }
    {
      top(nv);
      m_pv(nv - 1);
      ring_barrier();
      dma_rows(nv + 2, 0, e2);
      dma_rows(nv + 2, 1, e2);
      load_ids(nv + 6, e6);
      read_ids(nv + 3);
    }
  } else {
    // waves 4-7, iteration t: V(t-1), barrier, M(t); the loop below runs from
    // the M turn of t to the V turn of t (so a query issued after M(t) is
    // waited for at the end of the same pass)
    // entering pass t: ea, eb, ec = entries of blocks t, t+1, t+2; e3, e6 =
    // entries of blocks t+3 and t+6, loaded one pass ahead
    Ent ec, e3, e6;
    {
      const Ent e2 = ent(2);
      e3 = ent(3);
      e6 = ent(6);
      top(0);
      dma_rows(2, 0, e2);
      ring_barrier();
      m_s(0);
      dma_rows(2, 1, e2);
      load_ids(6, e6);
      read_ids(3);
      top(1);
      dma_rows(3, 0, e3);
      if (nv > 1 && is_first(eb)) {
        load_query(item_idx(eb));
        query_landed();
      }
      const Ent n3 = ent(4), n6 = ent(7);
      v_phase(ea.kb);
      ring_barrier();
      ea = eb;
      eb = e2;
      ec = e3;
      e3 = n3;
      e6 = n6;
    }
    for (int t = 1; t < nv; ++t) {
      const bool bnd = is_first(ea);
      const bool nq = t + 1 < nv && is_first(eb);
      m_both(t);
      dma_rows(t + 2, 1, ec);
      load_ids(t + 6, e6);
      read_ids(t + 3);
      top(t + 1);
      dma_rows(t + 3, 0, e3);
      if (bnd) {
        finish(cur);
        cur = item_idx(ea);
        setup(cur);
      }
      if (nq) {
        load_query(item_idx(eb));
        query_landed();
      }
      const Ent n3 = ent(t + 4), n6 = ent(t + 7);
      v_phase(ea.kb);
      ring_barrier();
      ea = eb;
      eb = ec;
      ec = e3;
      e3 = n3;
      e6 = n6;
    }
    m_pv(nv - 1);
    dma_rows(nv + 2, 1, ec);
    load_ids(nv + 6, ent(nv + 6));
    read_ids(nv + 3);
  }
  // drain the loads of blocks past the end before the LDS is reused
  wait_vm<0>();
  finish(cur);
}

// Sixteen FP8 E4M3 values (one 16-byte load) widened exactly to T: the two
// 16-byte chunks of 8 values each (values 0-7, then 8-15).
template <typename T>
__device__ __forceinline__ void fp8x16_widen(const u32x4 w, u32x4& c0, u32x4& c1) {
  uint32_t o[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (std::is_same<T, __bf16>::value) {
      o[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, false));
      o[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, true));
    } else {
      o[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[i], 1.0f, false));
      o[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[i], 1.0f, true));
    }
  }
  c0 = u32x4{o[0], o[1], o[2], o[3]};
  c1 = u32x4{o[4], o[5], o[6], o[7]};
}

// ----------------------------------------------------------------------------
// Key chunk: all q_len x group rows (<= 32) of one request and kv head over keys
// [kv_begin, kv_end). Wave w takes 32-key steps w, w+8, ... Each wave load
// instruction covers 4 whole 256-byte rows (16 lanes per row); K and V go to
// the wave's own LDS blocks, from which the K operand and the V^T operand are
// read. The next step's rows are in flight while the current step computes,
// and the page indices are fetched one step further ahead.
// Wave states merge in LDS; split chunks merge through the float workspace.
// kCols 32: the rows are one 32-wide MFMA column block (32x32x16 MFMAs).
// kCols 16: at most 16 rows; 16x16x32 MFMAs, half the MFMA and softmax work per
// key. Score block b (16 keys) holds key 16b + 4(lane/16) + j in accumulator j of
// column lane % 16; the 8 keys of a lane, in that order, are also the k-slots of
// its P^T operand (slot 8(lane/16) + e), so the V^T operand reads keys 4(lane/16)
// + [0,4) and 16 + 4(lane/16) + [0,4); head dims go to lane group q = lane/16 as
// d = 32q + 8c + [0,8) in the c-th score MFMA.
// cc / carried: the loads of this chunk's first step when the previous chunk
// issued them (carried), and on return those of item next_idx (>= 0: the next
// item of the list, of the same kind) when the rows are 16-bit and the chunk
// has at most 16 query rows (the wider form has no registers to spare).
template <typename T, bool kFp8, int kCols>
__device__ __forceinline__ void chunk_item(PArg p, const RoleView& r, const RowGeom& rg, int kvh,
                           int row0, int kv_begin, int kv_end, int split, int grp, char* lds, int wave_s,
                           ChunkCarry& cc, bool& carried, int next_idx) {
  using V8 = typename Dt<T>::v8;
  // the thread index, rebuilt from the wave (scalar) and the lane count, so the
  // hardware's thread-id register need not live through the whole launch; and
  // opaque to the compiler, so nothing derived from it is computed once for
  // all items of the workgroup and held in registers
  int tid = wave_s * 64 + (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63, wave = tid >> 6;
  const int r32 = lane & 31, hi = lane >> 5;
  const int q16 = lane >> 4;                       // 16-column mode: lane group
  const int col = kCols == 16 ? (lane & 15) : r32;   // this lane's row of the item
  const int g = p.group_size;
  // this item's rows: row0 .. row0 + rows - 1 of the request's q_len x group
  // rows (a row slice of at most 32 when the request has more)
  const int rows = min(kChunkRows, rg.qo_len * g - row0);
  const bool row_ok = col < rows;
  const int tok = row_ok ? (row0 + col) / g : 0;
  const int head = kvh * g + (row_ok ? (row0 + col) % g : 0);

  V8 qreg[8];
  if constexpr (kCols == 32) {
    load_q<T>(qreg, r, row_ok, rg.qo_start + tok, head, hi);
  } else {
    const T* qp = reinterpret_cast<const T*>(r.q) + (int64_t)(rg.qo_start + tok) * r.q_st +
                  (int64_t)head * r.q_sh + 32 * q16;
#pragma unroll
    for (int c = 0; c < 4; ++c) qreg[c] = __builtin_bit_cast(V8, row_ok ? ld16(qp + 8 * c) : u32x4{0, 0, 0, 0});
  }

  const int pdiag = rg.kv_len - rg.qo_len + tok;
  const int key_hi = min(r.causal ? pdiag : rg.kv_len - 1, kv_end - 1);
  const int key_lo = r.window_left >= 0 ? max(0, pdiag - r.window_left) : 0;
  const RowMask rm = row_mask(key_lo, key_hi);

  char* Kw = lds + wave * kWaveLds;
  char* Vw = Kw + kWaveKBytes;
  f32x16 o[4];
  f32x4 o16[8];
#pragma unroll
  for (int b = 0; b < 4; ++b) o[b] = f32x16{};
#pragma unroll
  for (int b = 0; b < 8; ++b) o16[b] = f32x4{};
  float m = kNegInf, l = 0.f;
  const float sl2 = r.scale_log2;

  // K operand offsets: 32 columns, MFMA c reads chunk 8 hi + c of row key_row(r32);
  // 16 columns, block b and MFMA c read chunk 4 q16 + c of row 16 b + lane % 16
  int koff[8];
  const char* vlane;
  if constexpr (kCols == 32) {
    const int krow = key_row(r32);
#pragma unroll
    for (int c = 0; c < 8; ++c) koff[c] = krow * kRowBytes + (((hi * 8 + c) ^ swz(krow)) << 4);
    vlane = Vw + vt_lane(lane);
  } else {
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int row = 16 * b + (lane & 15);
        koff[4 * b + c] = row * kRowBytes + (((4 * q16 + c) ^ swz(row)) << 4);
      }
    // V^T: lane i of group q addresses row 4q + i/4, dims 4(i%4) (+ block offset)
    vlane = Vw + (4 * q16 + ((lane & 15) >> 2)) * kVRowBytes + 8 * (lane & 3);
  }

  // the wave's first key and step count from the scalar wave index (uniform)
  const int first = kv_begin + kStepKeys * wave_s;
  const int n_steps = first < kv_end ? (kv_end - first + kWaves * kStepKeys - 1) / (kWaves * kStepKeys) : 0;
  // one step's scores, softmax and P.V from the wave's LDS blocks (keys kb..)
  auto compute16 = [&](int kb) __attribute__((always_inline)) {
    f32x4 s[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      s[b] = f32x4{};
#pragma unroll
      for (int c = 0; c < 4; ++c)
        s[b] = Dt<T>::mfma16(__builtin_bit_cast(V8, lds_ld16(Kw, koff[4 * b + c])), qreg[c], s[b]);
    }
    const int kq = kb + 4 * q16;
    if (__any((unsigned)(kb - rm.lo) > rm.span || (unsigned)(kb + kStepKeys - 1 - rm.lo) > rm.span)) {
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          s[b][j] = ((unsigned)(kq + 16 * b + j - rm.lo) <= rm.span) ? s[b][j] : kNegInf;
    }
    // column max over the lane's 8 keys and the other three lane groups
    float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                     fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const bool upd = (m == kNegInf) ? (mx != kNegInf) : ((mx - m) * sl2 > kRescaleThreshold);
    if (__any(upd)) {
      const float mn = upd ? mx : m;
      const float alpha = upd ? fast_exp2((m - mn) * sl2) : 1.f;
      l *= alpha;
#pragma unroll
      for (int b = 0; b < 8; ++b) o16[b] *= alpha;
      m = mn;
    }
    const float mu2 = (m == kNegInf) ? 0.f : m * sl2;
    V8 pb;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float e = fast_exp2(fmaf(s[b][j], sl2, -mu2));
        l += e;
        pb[4 * b + j] = (T)e;
      }
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      u32x2 part[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const LDS_AS char* pp = (const LDS_AS char*)vlane + 16 * h * kVRowBytes + db * 32;
        part[h] = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)pp));
      }
      const u32x4 w = {part[0][0], part[0][1], part[1][0], part[1][1]};
      o16[db] = Dt<T>::mfma16(__builtin_bit_cast(V8, w), pb, o16[db]);
    }
  };
  auto compute = [&](int kb) __attribute__((always_inline)) {
    if constexpr (kCols == 16) {
      compute16(kb);
      return;
    }
    f32x16 s[1];
    s[0] = f32x16{};
#pragma unroll
    for (int c = 0; c < 8; ++c)
      s[0] = Dt<T>::mfma(__builtin_bit_cast(V8, lds_ld16(Kw, koff[c])), qreg[c], s[0]);
    if (__any((unsigned)(kb - rm.lo) > rm.span || (unsigned)(kb + kStepKeys - 1 - rm.lo) > rm.span)) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int kidx = kb + acc_key(j, hi);
        s[0][j] = ((unsigned)(kidx - rm.lo) <= rm.span) ? s[0][j] : kNegInf;
      }
    }
    V8 pb[1][2];
    softmax_step<T, 1>(s, sl2, m, l, o, pb);
#pragma unroll
    for (int mp = 0; mp < 2; ++mp)
#pragma unroll
      for (int db = 0; db < 4; ++db)
        o[db] = Dt<T>::mfma(vt_operand<V8>(vlane, 16 * mp, db * 32), pb[0][mp], o[db]);
  };
  auto step_kb = [&](int i) { return first + kWaves * kStepKeys * i; };

  if constexpr (!kFp8) {
    // loads: instruction c moves row 4c + (lane >> 4) of the step, slot lane & 15
    const int ld_row = lane >> 4, ld_slot = lane & 15;
    uint32_t (&pidx)[8] = cc.pidx;
    u32x4 (&kst)[8] = cc.kst;
    u32x4 (&vst)[8] = cc.vst;
    const KeySrc cur{r.k, r.v, r.indices, r.kv_sp_b, r.kv_st_b, rg.page_start, first, kv_end - 1};
    // the next item, when its rows load the same way and this wave has keys in it
    KeySrc nxt = cur;
    bool has_next = false;
    if (kCols == 16 && next_idx >= 0) {
      CI32* it = plan_words(image_region(p, kHdrItems)) + next_idx * kItemWords;
      const int nfirst = it[5] + kStepKeys * wave_s;
      if (nfirst < it[6]) {
        const RoleView r2 = pick_role(p, it[0] & kFlagRole, it[2]);
        CI32* td = plan_words(image_region(p, kHdrTdesc)) + next_idx * kTdescWords;
        nxt = KeySrc{r2.k, r2.v, r2.indices, r2.kv_sp_b, r2.kv_st_b, td[3], nfirst, it[6] - 1};
        has_next = true;
      }
    }
    // rows past the chunk's end repeat its last row (masked to zero weight)
    auto pages_of = [&](const KeySrc& s, int i) __attribute__((always_inline)) {
      const int kb = s.first + kWaves * kStepKeys * i;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int key = min(kb + 4 * c + ld_row, s.last);
        const int pg = p.page_shift >= 0 ? (key >> p.page_shift) : key / p.page_size;
        pidx[c] = s.indices ? (uint32_t)s.indices[s.page_start + pg] : (uint32_t)(s.page_start + pg);
      }
    };
    auto rows_of = [&](const KeySrc& s, int i) __attribute__((always_inline)) {
      const int kb = s.first + kWaves * kStepKeys * i;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int key = min(kb + 4 * c + ld_row, s.last);
        const int slot = p.page_shift >= 0 ? (key & (p.page_size - 1)) : key % p.page_size;
        const uint64_t off = (uint64_t)pidx[c] * s.sp_b + (uint32_t)slot * s.st_b;
        kst[c] = ld16(s.k + off + ((ld_slot ^ swz(4 * c + ld_row)) << 4));
        vst[c] = ld16(s.v + off + (ld_slot << 4));
      }
    };
    if (!carried && n_steps > 0) {
      pages_of(cur, 0);
      rows_of(cur, 0);
      if (n_steps > 1) pages_of(cur, 1);
    }
    for (int i = 0; i < n_steps; ++i) {
      // this step's rows to the wave's blocks; the previous step's reads of them
      // are ordered before these writes (LDS runs a wave's requests in order)
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        lds_st16(Kw, (4 * c + ld_row) * kRowBytes + (ld_slot << 4), kst[c]);
        lds_st16(Vw, (4 * c + ld_row) * kVRowBytes + (ld_slot << 4), vst[c]);
      }
      if (i + 1 < n_steps) {
        rows_of(cur, i + 1);
        if (i + 2 < n_steps)
          pages_of(cur, i + 2);
        else if (has_next)
          pages_of(nxt, 0);   // a step ahead, as within the chunk
      }
      compute(step_kb(i));
    }
    carried = has_next;
    if (has_next) {
      if (n_steps < 2) pages_of(nxt, 0);
      rows_of(nxt, 0);
      pages_of(nxt, 1);
    }
  } else {
    // FP8 rows are 128 bytes: instruction c moves row 8c + (lane >> 3) of the
    // step, bytes 16 (lane & 7) .. +16, widened to two 16-byte chunks of T in the
    // same LDS layout. A step is half the bytes, so two steps stay in flight
    // (register sets a and b, steps alternating), page ids two steps ahead.
    // Every load here is unconditional, so the compiler can count the ones in
    // flight (a load under a branch, or a register a load targets being
    // overwritten on one path, makes it wait for all of them): FP8 pools always
    // come with a page table, and loads past the chunk repeat its last row
    // (cache hits, never computed on).
    const int ld_row = lane >> 3, ld_part = lane & 7;
    const int32_t* const id_base = r.indices + rg.page_start;
    uint32_t pa[4], pb2[4];
    u32x4 ka[4], va[4], kb2[4], vb2[4];
    auto load_pages = [&](int i, uint32_t (&pi)[4]) {
      const int kb = step_kb(i);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int key = min(kb + 8 * c + ld_row, kv_end - 1);
        const int pg = p.page_shift >= 0 ? (key >> p.page_shift) : key / p.page_size;
        pi[c] = (uint32_t)id_base[pg];
      }
    };
    auto load_rows = [&](int i, const uint32_t (&pi)[4], u32x4 (&kk)[4], u32x4 (&vv)[4]) {
      const int kb = step_kb(i);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint64_t off = row_off(r, p, pi[c], min(kb + 8 * c + ld_row, kv_end - 1)) + (ld_part << 4);
        kk[c] = ld16(r.k + off);
        vv[c] = ld16(r.v + off);
      }
    };
    auto store_rows = [&](const u32x4 (&kk)[4], const u32x4 (&vv)[4]) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int row = 8 * c + ld_row;
        u32x4 k0, k1, v0, v1;
        fp8x16_widen<T>(kk[c], k0, k1);
        fp8x16_widen<T>(vv[c], v0, v1);
        lds_st16(Kw, row * kRowBytes + (((2 * ld_part) ^ swz(row)) << 4), k0);
        lds_st16(Kw, row * kRowBytes + (((2 * ld_part + 1) ^ swz(row)) << 4), k1);
        lds_st16(Vw, row * kVRowBytes + ((2 * ld_part) << 4), v0);
        lds_st16(Vw, row * kVRowBytes + ((2 * ld_part + 1) << 4), v1);
      }
    };
    if (n_steps > 0) {
      // the prologue leaves the loads in flight in the loop's own order (rows
      // of a step, then the page ids two steps on), so the compiler's count of
      // them at the loop head is exact
      load_pages(0, pa);
      load_pages(1, pb2);
      load_rows(0, pa, ka, va);
      load_pages(2, pa);
      load_rows(1, pb2, kb2, vb2);
      load_pages(3, pb2);
      for (int i = 0; i < n_steps; i += 2) {
        store_rows(ka, va);
        load_rows(i + 2, pa, ka, va);
        load_pages(i + 4, pa);
        compute(step_kb(i));
        store_rows(kb2, vb2);
        load_rows(i + 3, pb2, kb2, vb2);
        load_pages(i + 5, pb2);
        if (i + 1 < n_steps) compute(step_kb(i + 1));
      }
    }
    carried = false;
  }
  if constexpr (kCols == 32) {
    l = xhalf_sum(l);
  } else {
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
  }

  // ---- merge the wave states in LDS
  __syncthreads();
  float* sm_m = reinterpret_cast<float*>(lds);    // [waves][32]
  float* sm_l = sm_m + kWaves * 32;               // [waves][32]
  float* accs = sm_l + kWaves * 32;               // 4 x [128 d][32 rows]
  int* sm_flag = reinterpret_cast<int*>(accs + 4 * kHeadDim * 32);
  // wave maxima in scaled (base-2) units
  const float m2 = (m == kNegInf) ? kNegInf : m * sl2;
  // one lane per row writes the row statistics: lane half 0 (32 columns) or
  // lane group 0 (16 columns)
  const bool stat_lane = kCols == 32 ? hi == 0 : q16 == 0;
  if (stat_lane) sm_m[wave * 32 + col] = m2;
  __syncthreads();
  float M = kNegInf;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w * 32 + col]);
  const float sc = (M == kNegInf) ? 0.f : fast_exp2(m2 - M);
  if (stat_lane) sm_l[wave * 32 + col] = l * sc;
  // waves w and w + 4 sum into partial sum w % 4 ([d][32 rows]; 16 columns
  // fill rows 0-15)
  float* acc = accs + (wave & 3) * kHeadDim * 32;
  auto put = [&](bool add) __attribute__((always_inline)) {
    if constexpr (kCols == 32) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          float& a = acc[(db * 32 + acc_d(j, hi)) * 32 + r32];
          a = add ? a + o[db][j] * sc : o[db][j] * sc;
        }
    } else {
#pragma unroll
      for (int db = 0; db < 8; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float& a = acc[(16 * db + 4 * q16 + j) * 32 + col];
          a = add ? a + o16[db][j] * sc : o16[db][j] * sc;
        }
    }
  };
  if (wave < 4) put(false);
  __syncthreads();
  if (wave >= 4) put(true);
  __syncthreads();

  // final stage on the first 256 threads: row threadIdx / 8, 16 dims each
  const int frow = (tid >> 3) & 31, d0 = (tid & 7) * 16;
  const bool fok = tid < 256 && frow < rows;
  const int ftok = fok ? (row0 + frow) / g : 0;
  const int fhead = kvh * g + (fok ? (row0 + frow) % g : 0);
  const int64_t out_row = (int64_t)(rg.qo_start + ftok);
  T* op = reinterpret_cast<T*>(r.out) + out_row * r.o_st + (int64_t)fhead * r.o_sh + d0;
  float* lse_p = r.lse ? r.lse + out_row * p.num_qo_heads + fhead : nullptr;
  const float sink_l2 = p.sinks ? p.sinks[fhead] * kLog2e : 0.f;

  if (fok) {
    float Mr = kNegInf, L = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      Mr = fmaxf(Mr, sm_m[w * 32 + frow]);
      L += sm_l[w * 32 + frow];
    }
    const float lse_r = L > 0.f ? Mr + fast_log2(L) : kNegInf;
    float vals[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = (d0 + i) * 32 + frow;
      vals[i] = (accs[e] + accs[kHeadDim * 32 + e]) + (accs[2 * kHeadDim * 32 + e] + accs[3 * kHeadDim * 32 + e]);
    }
    if (grp < 0) {
      const float mu = (Mr == kNegInf) ? 0.f : Mr;
      float den = L;
      if (p.sinks) den += fast_exp2(sink_l2 - mu);
      const float inv = den > 0.f ? r.v_scale / den : 0.f;
      V8 w0, w1;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        w0[i] = (T)(vals[i] * inv);
        w1[i] = (T)(vals[8 + i] * inv);
      }
      __builtin_nontemporal_store(__builtin_bit_cast(u32x4, w0), reinterpret_cast<u32x4*>(op));
      __builtin_nontemporal_store(__builtin_bit_cast(u32x4, w1), reinterpret_cast<u32x4*>(op) + 1);
      if (lse_p && (tid & 7) == 0) __builtin_nontemporal_store(lse_r, lse_p);
    } else {
      const int first_slot = image_region(p, kHdrGroups)[grp * kGroupWords + 1];
      float* slot = p.partials + (int64_t)(first_slot + split) * kSlotFloats;
      const float inv = L > 0.f ? 1.f / L : 0.f;
      // die-coherent stores (sc1: relaxed atomics at agent scope), so the last
      // workgroup of the group reads them from any die without an L2 writeback
      float* dst = slot + frow * kHeadDim + d0;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        __hip_atomic_store(dst + i, vals[i] * inv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if ((tid & 7) == 0)
        __hip_atomic_store(slot + kChunkRows * kHeadDim + frow, lse_r, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (grp < 0) return;

  // ---- split-KV: the last workgroup of the group merges every partial state
  const int32_t* groups = image_region(p, kHdrGroups);
  const int n_splits = groups[grp * kGroupWords + 0];
  const int first_slot = groups[grp * kGroupWords + 1];
  // Publication without fences: every partial went out with a die-coherent
  // store; each thread waits until its stores have completed, the workgroup
  // syncs, and only then is the group's counter bumped. The last arriver reads
  // the partials with die-coherent loads. (An agent-scope release fence would
  // write back the die's whole L2, every key block of it included.)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) {
    const int prev = atomicAdd(image_region(p, kHdrCounters) + grp, 1);
    *sm_flag = (prev == n_splits - 1);
  }
  __syncthreads();
  if (!*sm_flag) return;
  auto ld_c = [](const float* a) { return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
  if (fok) {
    const float* base = p.partials + (int64_t)first_slot * kSlotFloats;
    // the partials' loads go out in batches (8 LSEs, then 4 states of 17 words),
    // so a merge of many splits waits for a few memory round trips, not one per
    // split; indices past the last split re-read it and weigh nothing
    const float* lse_col = base + kChunkRows * kHeadDim + frow;
    float Mx = kNegInf;
    for (int s = 0; s < n_splits; s += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = ld_c(lse_col + (int64_t)min(s + u, n_splits - 1) * kSlotFloats);
#pragma unroll
      for (int u = 0; u < 8; ++u) Mx = fmaxf(Mx, v[u]);
    }
    float acc16[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc16[i] = 0.f;
    float tot = 0.f;
    if (Mx != kNegInf) {
      for (int s = 0; s < n_splits; s += 4) {
        float lv[4], x[4][16];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float* sl = base + (int64_t)min(s + u, n_splits - 1) * kSlotFloats;
          lv[u] = ld_c(sl + kChunkRows * kHeadDim + frow);
#pragma unroll
          for (int i = 0; i < 16; ++i) x[u][i] = ld_c(sl + frow * kHeadDim + d0 + i);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float w = s + u < n_splits ? fast_exp2(lv[u] - Mx) : 0.f;
          tot += w;
#pragma unroll
          for (int i = 0; i < 16; ++i) acc16[i] += w * x[u][i];
        }
      }
    }
    const float L = tot > 0.f ? Mx + fast_log2(tot) : kNegInf;
    float inv = tot > 0.f ? r.v_scale / tot : 0.f;
    if (p.sinks && tot > 0.f) inv = inv / (1.f + fast_exp2(sink_l2 - L));
    V8 w0, w1;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      w0[i] = (T)(acc16[i] * inv);
      w1[i] = (T)(acc16[8 + i] * inv);
    }
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, w0), reinterpret_cast<u32x4*>(op));
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, w1), reinterpret_cast<u32x4*>(op) + 1);
    if (lse_p && (tid & 7) == 0) __builtin_nontemporal_store(L, lse_p);
  }
  if (tid == 0) atomicExch(image_region(p, kHdrCounters) + grp, 0);
}

// Kind of a key-chunk item: bit 1 FP8 rows, bit 0 at most 16 rows (16x16x32
// MFMAs).
__device__ __forceinline__ int chunk_kind(PArg p, int idx) {
  CI32* it = plan_words(image_region(p, kHdrItems)) + idx * kItemWords;
  CI32* td = plan_words(image_region(p, kHdrTdesc)) + idx * kTdescWords;   // request fields
  const bool fp8 = (it[0] & kFlagRole) && p.role[1].kv_fp8;
  const bool narrow = td[1] * p.group_size - it[3] <= 16;   // rows of the item (slice)
  return 2 * fp8 + narrow;
}

// Key-chunk items idx0, idx0 + 1, ... (below end) while they are of this kind,
// the first step's loads of each issued in the previous one's tail. Returns
// how many ran (at least one).
template <typename T, bool kFp8, int kCols>
__device__ __forceinline__ int chunk_items(PArg p, int idx0, int end, char* lds, int wave_s) {
  constexpr int kKind = 2 * kFp8 + (kCols == 16);
  ChunkCarry cc;
  bool carried = false;
  int idx = idx0;
  for (;;) {
    const int next = idx + 1 < end && chunk_kind(p, idx + 1) == kKind ? idx + 1 : -1;
    CI32* it = plan_words(image_region(p, kHdrItems)) + idx * kItemWords;
    const int flags = it[0];
    const int kvh = it[2], kv_begin = it[5], kv_end = it[6], grp = it[7];
    const RoleView r = pick_role(p, flags & kFlagRole, kvh);
    CI32* td = plan_words(image_region(p, kHdrTdesc)) + idx * kTdescWords;   // request fields
    const RowGeom rg{td[0], td[1], td[2], td[3]};
    chunk_item<T, kFp8, kCols>(p, r, rg, kvh, it[3], kv_begin, kv_end, flags >> kSplitShift, grp, lds, wave_s,
                               cc, carried, next);
    if (next < 0) break;
    __syncthreads();   // the item is done with the LDS
    idx = next;
  }
  return idx + 1 - idx0;
}

// One persistent workgroup per CU runs its static list from the plan: its key
// chunks one after another, and its query tiles as one block stream (chunks
// first or last, as the plan says). Then it takes key chunks from the shared
// pool, one at a time through an atomic counter, until the pool is empty; the
// last workgroup to find it empty puts the counters back to zero for the next
// launch.
template <typename T>
__global__ __launch_bounds__(kThreads, 1) void pod_grid_kernel(Params) {
  PArg p = *(const __attribute__((address_space(4))) Params*)__builtin_amdgcn_kernarg_segment_ptr();
  // the query tiles' ring slots, or one 18 KB part per key-chunk wave
  __shared__ __attribute__((aligned(16))) char lds[kLdsMain];
  // page-id ring of the query tiles: 4 slots x 8 waves x 64 words
  __shared__ __attribute__((aligned(16))) char ids[kRingSlots * kIdSlot];
  // sink logits for the query tiles' normalisation
  __shared__ __attribute__((aligned(16))) float sink_lds[kMaxSinkHeads];
  __shared__ int pool_slot;
  // destination of the block-table prefetch
  __shared__ __attribute__((aligned(16))) char pf_lds[256];
  const int wave_s = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  CI32* wg = plan_words(image_region(p, kHdrWgs)) + blockIdx.x * kWgWords;
  const int first_item = wg[0], n_tiles = wg[1], n_chunks = wg[2];
  const int first_blk = wg[3], n_blk = wg[4];
  const bool chunks_first = wg[5] != 0;
  // the items idx .. end - 1 of the list while they are of one kind; returns
  // how many ran
  auto run_chunk_items = [&](int idx, int end) __attribute__((always_inline)) {
    switch (chunk_kind(p, idx)) {
      case 3: return chunk_items<T, true, 16>(p, idx, end, lds, wave_s);
      case 2: return chunk_items<T, true, 32>(p, idx, end, lds, wave_s);
      case 1: return chunk_items<T, false, 16>(p, idx, end, lds, wave_s);
      default: return chunk_items<T, false, 32>(p, idx, end, lds, wave_s);
    }
  };
  auto run_chunks = [&]() __attribute__((always_inline)) {
    const int c0 = first_item + n_tiles;
    for (int j = 0; j < n_chunks;) {
      __syncthreads();   // the previous item is done with the LDS
      j += run_chunk_items(c0 + j, c0 + n_chunks);
    }
  };
  if (chunks_first) run_chunks();
  if (n_tiles > 0) {
    __syncthreads();
    const int32_t* ttd = image_region(p, kHdrTdesc) + (int64_t)first_item * kTdescWords;
    const int pre_tiles = wg[6];
    const int32_t* tb = image_region(p, kHdrBlocks) + (int64_t)first_blk * kBlockWords;
    // one block stream per role: the prefill tiles, then the decode tiles
    const int pre_blk = wg[7];
    for (int role = 0; role < 2; ++role) {
      const int b0 = role ? pre_blk : 0, nb = role ? n_blk - pre_blk : pre_blk;
      if (nb == 0) continue;
      if (role && pre_blk) __syncthreads();
      const int t0 = role ? pre_tiles : 0, nt = role ? n_tiles - pre_tiles : pre_tiles;
      const int32_t* tbr = tb + (int64_t)b0 * kBlockWords;
      if (p.page_shift >= 0 && p.role[role].indices != nullptr)
        tile_stream<T, true, 1>(p, role, ttd, t0, nt, tbr, nb, lds, ids, sink_lds, pf_lds);
      else if (p.page_shift >= 0)
        tile_stream<T, true, 0>(p, role, ttd, t0, nt, tbr, nb, lds, ids, sink_lds, pf_lds);
      else
        tile_stream<T, false, 2>(p, role, ttd, t0, nt, tbr, nb, lds, ids, sink_lds, pf_lds);
    }
  }
  if (!chunks_first) run_chunks();
  const int pool_count = hdr_word(p, kHdrPoolCount);
  if (pool_count > 0) {
    int32_t* queue = image_region(p, kHdrQueue);
    for (;;) {
      __syncthreads();   // the previous item is done with the LDS and pool_slot
      if (threadIdx.x == 0) pool_slot = atomicAdd(queue, 1);
      __syncthreads();
      const int j = __builtin_amdgcn_readfirstlane(pool_slot);
      if (j >= pool_count) break;
      const int idx = hdr_word(p, kHdrPoolFirst) + j;
      run_chunk_items(idx, idx + 1);
    }
    // every workgroup has taken its last (empty) turn before it counts itself
    // done, so the last one can clear both counters
    if (threadIdx.x == 0 && atomicAdd(queue + 1, 1) == (int)gridDim.x - 1) {
      atomicExch(queue, 0);
      atomicExch(queue + 1, 0);
    }
  }
}

}  // namespace

int static_scratch(int device, void** ptr) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  if (device < 0 || device >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[device]) {
    // with `device` current: this device's copy of the array
    void* a = nullptr;
    const hipError_t e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    if (!a) return (int)hipErrorInvalidSymbol;
    addr[device] = a;
  }
  *ptr = addr[device];
  return (int)hipSuccess;
}

int launch_pod_grid(const Params& p, int dtype, int grid, void* stream, void* done_event) {
  if (grid <= 0) return (int)hipSuccess;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipEvent_t done = reinterpret_cast<hipEvent_t>(done_event);
  if (!done) {   // a plain dispatch (capturable into a graph)
    if (dtype == POD_DTYPE_BF16)
      hipLaunchKernelGGL(pod_grid_kernel<__bf16>, dim3(grid), dim3(kThreads), 0, s, p);
    else
      hipLaunchKernelGGL(pod_grid_kernel<_Float16>, dim3(grid), dim3(kThreads), 0, s, p);
    return (int)hipGetLastError();
  }
  // the completion event rides on the dispatch itself (no separate marker)
  if (dtype == POD_DTYPE_BF16)
    hipExtLaunchKernelGGL(pod_grid_kernel<__bf16>, dim3(grid), dim3(kThreads), 0, s, nullptr, done, 0, p);
  else
    hipExtLaunchKernelGGL(pod_grid_kernel<_Float16>, dim3(grid), dim3(kThreads), 0, s, nullptr, done, 0, p);
  return (int)hipGetLastError();
}

}  // namespace pod
