// Fused Prefill-On-Decode paged attention for gfx950 (MI355X, CDNA4).
//
// One launch runs every item of the planner's work list: query tiles (prefill
// style: up to 128 rows share each staged K/V block) and key chunks (decode
// style: the q_len x group rows of one request and kv head share every K/V row
// read from HBM, the keys are split over the 4 waves and over workgroups).
// This is the "prefill and decode in one launch" idea of the POD article
// (www.dpshk.com/news/5405057, "POD 是什么"), built for wave64 and MFMA.
//
// Math per row (cuDNN backend article www.gsyq.cn/news/452757, "LSE 契约" and
// "Decode 能力矩阵与参数"): scores s_j = sm_scale * q.k_j over the row's valid
// keys, O = sum_j softmax_j v_j with an optional sink logit in the
// denominator, lse = log2 sum_j exp(s_j). Work is done in the base-2 domain:
// t_j = s_j * log2(e), online max / sum with exp2, and partial states over
// disjoint key ranges merge as L = log2 sum 2^lse_k, O = sum 2^(lse_k - L) O_k.
//
// MFMA formulation (v_mfma_f32_32x32x16_{bf16,f16}):
//   S^T[key][row] = K[key][:] . Q[row][:]   A = K rows, B = Q^T (in registers)
//   O^T[d][row]  += V^T[d][key] . P^T[key][row]   A = V^T (LDS), B = P^T (registers)
// The accumulator keeps one query row per lane column, so the softmax row
// statistics are per-lane scalars plus one exchange between the two lane
// halves. K rows are assigned to MFMA rows with bits 2 and 3 of the row index
// swapped, which makes the score accumulator registers of each lane half hold
// 8 consecutive keys: the P^T operand then comes straight from the
// accumulators, and V^T is read as 16 contiguous bytes per lane.
#include <hip/hip_runtime.h>

#include <math.h>

#include "pod_internal.h"

namespace pod {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

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
};
template <>
struct Dt<_Float16> {
  using v8 = f16x8;
  using v4 = f16x4;
  static __device__ __forceinline__ f32x16 mfma(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

// LDS geometry (element counts; rows padded by 8 elements = 16 bytes)
constexpr int kTileKeys = 64;                 // keys per staged block of a query tile
constexpr int kKsStride = kHeadDim + 8;       // K block [64 keys][136]
constexpr int kVtStride = kTileKeys + 8;      // V^T block [128 d][72]
constexpr int kChunkKeys = 32;                // keys per wave step of a key chunk
constexpr int kCvStride = kChunkKeys + 8;     // per-wave V^T block [128 d][40]
constexpr int kTileLds = (kTileKeys * kKsStride + kHeadDim * kVtStride) * 2;
constexpr int kChunkLds = 4 * kHeadDim * kCvStride * 2;
constexpr int kMergeLds = (4 * 32 * 2 + 2 * kHeadDim * 32) * 4 + 16;
constexpr int kLdsBytes = kTileLds > kChunkLds ? (kTileLds > kMergeLds ? kTileLds : kMergeLds)
                                               : (kChunkLds > kMergeLds ? kChunkLds : kMergeLds);

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// MFMA row m of the score block holds key swap_bits23(m) of the 32-key group.
__device__ __forceinline__ int key_row(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}
// key (within a 32-key group) held by score accumulator j of lane half hi
__device__ __forceinline__ int acc_key(int j, int hi) { return 16 * (j >> 3) + 8 * hi + (j & 7); }
// head-dim index held by output accumulator j (of a 32-wide d block) of lane half hi
__device__ __forceinline__ int acc_d(int j, int hi) { return 8 * (j >> 2) + 4 * hi + (j & 3); }

template <typename T>
__device__ __forceinline__ u32x4 ld16(const T* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

struct RowGeom {
  int qo_start, qo_len, kv_len, page_start;
};

struct RoleView {
  const void* q;
  int64_t q_st, q_sh;
  const void* k;
  const void* v;
  int64_t kv_sp, kv_st, kv_sh;
  const int32_t* indices;
  void* out;
  int64_t o_st, o_sh;
  float* lse;
  float scale_log2;
  int causal, window_left;
};

__device__ __forceinline__ RoleView pick_role(const Params& p, int role) {
  const RoleParams& a = p.role[0];
  const RoleParams& b = p.role[1];
  RoleView r;
  r.q = role ? b.q : a.q;
  r.q_st = role ? b.q_st : a.q_st;
  r.q_sh = role ? b.q_sh : a.q_sh;
  r.k = role ? b.k : a.k;
  r.v = role ? b.v : a.v;
  r.kv_sp = role ? b.kv_sp : a.kv_sp;
  r.kv_st = role ? b.kv_st : a.kv_st;
  r.kv_sh = role ? b.kv_sh : a.kv_sh;
  r.indices = role ? b.indices : a.indices;
  r.out = role ? b.out : a.out;
  r.o_st = role ? b.o_st : a.o_st;
  r.o_sh = role ? b.o_sh : a.o_sh;
  r.lse = role ? b.lse : a.lse;
  r.scale_log2 = role ? b.scale_log2 : a.scale_log2;
  r.causal = role ? b.causal : a.causal;
  r.window_left = role ? b.window_left : a.window_left;
  return r;
}

// Element offset of (logical key, kv head) in a role's pool.
__device__ __forceinline__ int64_t kv_offset(const RoleView& r, int page_size, int page_start,
                                             int key, int kvh) {
  int pg = key / page_size;
  int slot = key - pg * page_size;
  int64_t page = r.indices ? (int64_t)r.indices[page_start + pg] : (int64_t)(page_start + pg);
  return page * r.kv_sp + (int64_t)slot * r.kv_st + (int64_t)kvh * r.kv_sh;
}

// Load the Q^T operand of one row: lane half hi holds d = hi*64 + c*8 + [0,8) for MFMA c.
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

// Online-softmax update for one block of score accumulators (base-2 domain).
// s: raw scores (already masked to -inf); returns P as operand vectors.
template <typename T, int NB>
__device__ __forceinline__ void softmax_step(f32x16 (&s)[NB], float& m, float& l,
                                             f32x16 (&o)[4], typename Dt<T>::v8 (&pb)[NB][2]) {
  float mx = kNegInf;
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int j = 0; j < 16; ++j) mx = fmaxf(mx, s[b][j]);
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float mn = fmaxf(m, mx);
  const float mu = (mn == kNegInf) ? 0.f : mn;
  const float alpha = fast_exp2(m - mu);
  l *= alpha;
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int j = 0; j < 16; ++j) o[b][j] *= alpha;
  m = mn;
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float e = fast_exp2(s[b][8 * h + i] - mu);
        l += e;
        pb[b][h][i] = (T)e;
      }
}

// ----------------------------------------------------------------------------
// Query tile: up to 128 rows (tokens x group heads) of one request and kv head,
// keys [kv_begin, kv_end) in blocks of 64 staged in LDS by all 4 waves.
template <typename T>
__device__ void tile_item(const Params& p, const RoleView& r, const RowGeom& rg, int kvh, int tok0,
                          int ntok, int kv_begin, int kv_end, char* smem) {
  using V8 = typename Dt<T>::v8;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r32 = lane & 31, hi = lane >> 5;
  const int g = p.group_size;
  const int rows = ntok * g;
  const int row = wave * 32 + r32;
  const bool row_ok = row < rows;
  const int tok = tok0 + (row_ok ? row / g : 0);
  const int head = kvh * g + (row_ok ? row % g : 0);

  V8 qreg[8];
  load_q<T>(qreg, r, row_ok, rg.qo_start + tok, head, hi);

  const int pdiag = rg.kv_len - rg.qo_len + tok;
  const int key_hi = r.causal ? pdiag : rg.kv_len - 1;
  const int key_lo = r.window_left >= 0 ? max(0, pdiag - r.window_left) : 0;

  T* Ks = reinterpret_cast<T*>(smem);
  T* Vt = Ks + kTileKeys * kKsStride;
  f32x16 o[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) o[b] = f32x16{};
  float m = kNegInf, l = 0.f;
  const float sl2 = r.scale_log2;
  const int krow = key_row(r32);
  const T* kbase = reinterpret_cast<const T*>(r.k);
  const T* vbase = reinterpret_cast<const T*>(r.v);

  for (int kb = kv_begin; kb < kv_end; kb += kTileKeys) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = threadIdx.x + kThreads * i;
      const int key = idx >> 4, ch = idx & 15;
      const int kidx = kb + key;
      u32x4 kx = {0, 0, 0, 0}, vx = {0, 0, 0, 0};
      if (kidx < kv_end) {
        const int64_t off = kv_offset(r, p.page_size, rg.page_start, kidx, kvh) + ch * 8;
        kx = ld16(kbase + off);
        vx = ld16(vbase + off);
      }
      *reinterpret_cast<u32x4*>(Ks + key * kKsStride + ch * 8) = kx;
      V8 ve = __builtin_bit_cast(V8, vx);
#pragma unroll
      for (int j = 0; j < 8; ++j) Vt[(ch * 8 + j) * kVtStride + key] = ve[j];
    }
    __syncthreads();

    f32x16 s[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      s[h] = f32x16{};
      const T* kr = Ks + (h * 32 + krow) * kKsStride + hi * 64;
#pragma unroll
      for (int c = 0; c < 8; ++c)
        s[h] = Dt<T>::mfma(__builtin_bit_cast(V8, ld16(kr + c * 8)), qreg[c], s[h]);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int kidx = kb + h * 32 + acc_key(j, hi);
        const bool ok = kidx >= key_lo && kidx <= key_hi && kidx < kv_end;
        s[h][j] = ok ? s[h][j] * sl2 : kNegInf;
      }
    V8 pb[2][2];
    softmax_step<T, 2>(s, m, l, o, pb);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int mp = 0; mp < 2; ++mp)
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const T* vp = Vt + (db * 32 + r32) * kVtStride + h * 32 + 16 * mp + 8 * hi;
          o[db] = Dt<T>::mfma(__builtin_bit_cast(V8, ld16(vp)), pb[h][mp], o[db]);
        }
  }
  l += __shfl_xor(l, 32);

  if (row_ok) {
    const float mu = (m == kNegInf) ? 0.f : m;
    float den = l;
    if (p.sinks) den += fast_exp2(p.sinks[head] * kLog2e - mu);
    const float inv = den > 0.f ? 1.f / den : 0.f;
    T* op = reinterpret_cast<T*>(r.out) + (int64_t)(rg.qo_start + tok) * r.o_st +
            (int64_t)head * r.o_sh;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        typename Dt<T>::v4 w;
#pragma unroll
        for (int c = 0; c < 4; ++c) w[c] = (T)(o[db][4 * a + c] * inv);
        *reinterpret_cast<u32x2*>(op + db * 32 + acc_d(4 * a, hi)) = __builtin_bit_cast(u32x2, w);
      }
    if (r.lse && hi == 0)
      r.lse[(int64_t)(rg.qo_start + tok) * p.num_qo_heads + head] =
          l > 0.f ? m + fast_log2(l) : kNegInf;
  }
}

// ----------------------------------------------------------------------------
// Key chunk: all q_len x group rows (<= 32) of one request and kv head over keys
// [kv_begin, kv_end). Wave w takes 32-key steps w, w+4, ...; K goes straight
// from HBM into MFMA operand registers, V through a per-wave transposed LDS
// block. Wave states merge in LDS; split chunks merge through the workspace.
template <typename T>
__device__ void chunk_item(const Params& p, const RoleView& r, const RowGeom& rg, int kvh,
                           int kv_begin, int kv_end, int split, int grp, char* smem) {
  using V8 = typename Dt<T>::v8;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r32 = lane & 31, hi = lane >> 5;
  const int g = p.group_size;
  const int rows = rg.qo_len * g;
  const bool row_ok = r32 < rows;
  const int tok = row_ok ? r32 / g : 0;
  const int head = kvh * g + (row_ok ? r32 % g : 0);

  V8 qreg[8];
  load_q<T>(qreg, r, row_ok, rg.qo_start + tok, head, hi);

  const int pdiag = rg.kv_len - rg.qo_len + tok;
  const int key_hi = r.causal ? pdiag : rg.kv_len - 1;
  const int key_lo = r.window_left >= 0 ? max(0, pdiag - r.window_left) : 0;

  T* Vt = reinterpret_cast<T*>(smem) + wave * (kHeadDim * kCvStride);
  f32x16 o[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) o[b] = f32x16{};
  float m = kNegInf, l = 0.f;
  const float sl2 = r.scale_log2;
  const int krow = key_row(r32);
  const T* kbase = reinterpret_cast<const T*>(r.k);
  const T* vbase = reinterpret_cast<const T*>(r.v);

  for (int kb = kv_begin + kChunkKeys * wave; kb < kv_end; kb += 4 * kChunkKeys) {
    V8 ak[8];
    {
      const int key = kb + krow;
      if (key < kv_end) {
        const T* kp = kbase + kv_offset(r, p.page_size, rg.page_start, key, kvh) + hi * 64;
#pragma unroll
        for (int c = 0; c < 8; ++c) ak[c] = __builtin_bit_cast(V8, ld16(kp + c * 8));
      } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) ak[c] = __builtin_bit_cast(V8, u32x4{0, 0, 0, 0});
      }
    }
    u32x4 vx[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int idx = lane + 64 * i;
      const int kidx = kb + (idx >> 4);
      vx[i] = kidx < kv_end
                  ? ld16(vbase + kv_offset(r, p.page_size, rg.page_start, kidx, kvh) + (idx & 15) * 8)
                  : u32x4{0, 0, 0, 0};
    }
    f32x16 s[1];
    s[0] = f32x16{};
#pragma unroll
    for (int c = 0; c < 8; ++c) s[0] = Dt<T>::mfma(ak[c], qreg[c], s[0]);

    // this wave's previous V^T reads are done before it is overwritten
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int idx = lane + 64 * i;
      const int key = idx >> 4, ch = idx & 15;
      V8 ve = __builtin_bit_cast(V8, vx[i]);
#pragma unroll
      for (int j = 0; j < 8; ++j) Vt[(ch * 8 + j) * kCvStride + key] = ve[j];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int kidx = kb + acc_key(j, hi);
      const bool ok = kidx >= key_lo && kidx <= key_hi && kidx < kv_end;
      s[0][j] = ok ? s[0][j] * sl2 : kNegInf;
    }
    V8 pb[1][2];
    softmax_step<T, 1>(s, m, l, o, pb);
#pragma unroll
    for (int mp = 0; mp < 2; ++mp)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const T* vp = Vt + (db * 32 + r32) * kCvStride + 16 * mp + 8 * hi;
        o[db] = Dt<T>::mfma(__builtin_bit_cast(V8, ld16(vp)), pb[0][mp], o[db]);
      }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  l += __shfl_xor(l, 32);

  // ---- merge the 4 wave states in LDS
  __syncthreads();
  float* sm_m = reinterpret_cast<float*>(smem);   // [4][32]
  float* sm_l = sm_m + 128;                       // [4][32]
  float* accA = sm_l + 128;                       // [128 d][32 rows]
  float* accB = accA + kHeadDim * 32;
  int* sm_flag = reinterpret_cast<int*>(accB + kHeadDim * 32);
  if (hi == 0) sm_m[wave * 32 + r32] = m;
  __syncthreads();
  float M = fmaxf(fmaxf(sm_m[r32], sm_m[32 + r32]), fmaxf(sm_m[64 + r32], sm_m[96 + r32]));
  const float sc = (M == kNegInf) ? 0.f : fast_exp2(m - M);
  if (hi == 0) sm_l[wave * 32 + r32] = l * sc;
  float* acc = (wave & 1) ? accB : accA;
  if (wave < 2) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[(db * 32 + acc_d(j, hi)) * 32 + r32] = o[db][j] * sc;
  }
  __syncthreads();
  if (wave >= 2) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[(db * 32 + acc_d(j, hi)) * 32 + r32] += o[db][j] * sc;
  }
  __syncthreads();

  const int frow = threadIdx.x >> 3, d0 = (threadIdx.x & 7) * 16;
  const bool fok = frow < rows;
  const int ftok = fok ? frow / g : 0;
  const int fhead = kvh * g + (fok ? frow % g : 0);
  const int64_t out_row = (int64_t)(rg.qo_start + ftok);
  T* op = reinterpret_cast<T*>(r.out) + out_row * r.o_st + (int64_t)fhead * r.o_sh + d0;
  float* lse_p = r.lse ? r.lse + out_row * p.num_qo_heads + fhead : nullptr;
  const float sink_l2 = p.sinks ? p.sinks[fhead] * kLog2e : 0.f;

  if (fok) {
    const float Mr = fmaxf(fmaxf(sm_m[frow], sm_m[32 + frow]), fmaxf(sm_m[64 + frow], sm_m[96 + frow]));
    const float L = sm_l[frow] + sm_l[32 + frow] + sm_l[64 + frow] + sm_l[96 + frow];
    const float lse_r = L > 0.f ? Mr + fast_log2(L) : kNegInf;
    float vals[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) vals[i] = accA[(d0 + i) * 32 + frow] + accB[(d0 + i) * 32 + frow];
    if (grp < 0) {
      const float mu = (Mr == kNegInf) ? 0.f : Mr;
      float den = L;
      if (p.sinks) den += fast_exp2(sink_l2 - mu);
      const float inv = den > 0.f ? 1.f / den : 0.f;
      V8 w0, w1;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        w0[i] = (T)(vals[i] * inv);
        w1[i] = (T)(vals[8 + i] * inv);
      }
      reinterpret_cast<u32x4*>(op)[0] = __builtin_bit_cast(u32x4, w0);
      reinterpret_cast<u32x4*>(op)[1] = __builtin_bit_cast(u32x4, w1);
      if (lse_p && (threadIdx.x & 7) == 0) *lse_p = lse_r;
    } else {
      const int first_slot = p.groups[grp * kGroupWords + 1];
      float* slot = p.partials + (int64_t)(first_slot + split) * kSlotFloats;
      const float inv = L > 0.f ? 1.f / L : 0.f;
      float4* dst = reinterpret_cast<float4*>(slot + frow * kHeadDim + d0);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        dst[i] = make_float4(vals[4 * i] * inv, vals[4 * i + 1] * inv, vals[4 * i + 2] * inv,
                             vals[4 * i + 3] * inv);
      if ((threadIdx.x & 7) == 0) slot[kChunkRows * kHeadDim + frow] = lse_r;
    }
  }
  if (grp < 0) return;

  // ---- split-KV: the last workgroup of the group merges every partial state
  const int n_splits = p.groups[grp * kGroupWords + 0];
  const int first_slot = p.groups[grp * kGroupWords + 1];
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const int prev = atomicAdd(&p.counters[grp], 1);
    *sm_flag = (prev == n_splits - 1);
  }
  __syncthreads();
  if (!*sm_flag) return;
  __threadfence();
  if (fok) {
    const float* base = p.partials + (int64_t)first_slot * kSlotFloats;
    float Mx = kNegInf;
    for (int s = 0; s < n_splits; ++s)
      Mx = fmaxf(Mx, base[(int64_t)s * kSlotFloats + kChunkRows * kHeadDim + frow]);
    float acc16[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc16[i] = 0.f;
    float tot = 0.f;
    if (Mx != kNegInf) {
      for (int s = 0; s < n_splits; ++s) {
        const float* sl = base + (int64_t)s * kSlotFloats;
        const float ls = sl[kChunkRows * kHeadDim + frow];
        const float w = fast_exp2(ls - Mx);
        tot += w;
        const float4* src = reinterpret_cast<const float4*>(sl + frow * kHeadDim + d0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 x = src[i];
          acc16[4 * i] += w * x.x;
          acc16[4 * i + 1] += w * x.y;
          acc16[4 * i + 2] += w * x.z;
          acc16[4 * i + 3] += w * x.w;
        }
      }
    }
    const float L = tot > 0.f ? Mx + fast_log2(tot) : kNegInf;
    float inv = tot > 0.f ? 1.f / tot : 0.f;
    if (p.sinks && tot > 0.f) inv = inv / (1.f + fast_exp2(sink_l2 - L));
    V8 w0, w1;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      w0[i] = (T)(acc16[i] * inv);
      w1[i] = (T)(acc16[8 + i] * inv);
    }
    reinterpret_cast<u32x4*>(op)[0] = __builtin_bit_cast(u32x4, w0);
    reinterpret_cast<u32x4*>(op)[1] = __builtin_bit_cast(u32x4, w1);
    if (lse_p && (threadIdx.x & 7) == 0) *lse_p = L;
  }
  if (threadIdx.x == 0) atomicExch(&p.counters[grp], 0);
}

template <typename T>
__global__ __launch_bounds__(kThreads, 2) void pod_grid_kernel(Params p) {
  __shared__ __attribute__((aligned(16))) char smem[kLdsBytes];
  const int32_t* it = p.items + (int64_t)blockIdx.x * kItemWords;
  const int flags = it[0];
  if (flags < 0) return;
  const int role = flags & kFlagRole;
  const int req = it[1], kvh = it[2], tok0 = it[3], ntok = it[4];
  const int kv_begin = it[5], kv_end = it[6], grp = it[7];
  const RoleView r = pick_role(p, role);
  const int32_t* rq = p.reqs + req * kReqWords;
  RowGeom rg{rq[0], rq[1], rq[2], rq[3]};
  if (flags & kFlagChunk)
    chunk_item<T>(p, r, rg, kvh, kv_begin, kv_end, flags >> kSplitShift, grp, smem);
  else
    tile_item<T>(p, r, rg, kvh, tok0, ntok, kv_begin, kv_end, smem);
}

}  // namespace

int launch_pod_grid(const Params& p, int dtype, int grid, void* stream) {
  if (grid <= 0) return (int)hipSuccess;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (dtype == POD_DTYPE_BF16)
    hipLaunchKernelGGL(pod_grid_kernel<__bf16>, dim3(grid), dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL(pod_grid_kernel<_Float16>, dim3(grid), dim3(kThreads), 0, s, p);
  return (int)hipGetLastError();
}

}  // namespace pod
