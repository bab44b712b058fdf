// libkvstore: KV-cache store kernels for MI355X (gfx950, CDNA4) and their C ABI.
//
// Two operations (declared, with argument rules, in include/kvstore.h):
//   * kvstore_copy      -- scatter copy of K/V rows into cache slots
//                          (sglang "kvcache.cuh", store_kvcache).
//   * kvstore_fp8_paged -- bf16/fp16 -> e4m3fn quantise fused with the paged
//                          [page, offset, head, dim] write
//                          (sglang "trtllm_fp8_kv_kernel.py",
//                          _fused_fp8_set_kv_buffer_kernel); also into e5m2
//                          caches, and with scales computed per token or per
//                          token and head (kvstore_fp8_paged_e5m2 / _dynamic).
//
// Both are pure data movement, bound by HBM bandwidth: no MFMA, and no LDS
// traffic for the rows (the copy allocates LDS only to cap its residency; the
// per-token dynamic store passes one scale per wave through it).
// Design points for CDNA4:
//   * one 64-lane wave per (token, K or V, slice of the row); each lane
//     loads 16 B per access (dwordx4), so one wave access
//     covers 1 KiB of consecutive row bytes; copy rows or pointers aligned
//     only to 8 or 4 bytes use 8- or 4-byte lanes, copy rows that need at
//     most 32 lanes are packed several to a wave, and copy launches of 6-48
//     MiB give each wave 8 tokens (see copy_tokens_per_wave);
//   * every load of a wave (all its 1 KiB chunks) is issued before the
//     index is needed: the source address does not depend on the index, so the
//     index fetch overlaps the data fetch instead of preceding it (the copy
//     kernels are written so that the compiler keeps that order; see
//     loaded() and indices_after_row_loads());
//   * the row base addresses are wave-uniform 64-bit values (scalar registers)
//     and the per-lane offset is a 32-bit vector register;
//   * copy: cache rows are written with non-temporal stores (which leave no
//     written lines behind for the next kernel), and residency is capped to
//     about 24 KiB of loads in flight per CU (12 waves of 2 KiB rows; see
//     copy_waves_per_cu): the rows land at scattered slots, and fewer
//     concurrent write streams measured faster;
//   * fp8: the quantised rows are written with the sc1 cache policy through a
//     per-row buffer descriptor, at full occupancy (the conversion needs the
//     latency hiding);
//   * a bad index does not trap: the wave skips its stores and records the
//     token in a per-device flag (smallest token, count).
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <atomic>
#include <mutex>

#include "kvstore.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;                     // lanes per wavefront (CDNA)
constexpr int kWavesPerBlock = 2;             // fp8 kernels
constexpr int kBlockThreads = kWave * kWavesPerBlock;
// fp8 kernel with dynamic scales: the block's waves store their scales with
// one instruction (per token, 4 waves: 17.97 us against 18.08 for 2 and 18.15
// for 8 on the 16384-token workload)
constexpr int kDynWavesPerBlock = 4;
constexpr int kCopyWavesPerBlock = 2;         // copy kernel
constexpr int kCopyBlockThreads = kWave * kCopyWavesPerBlock;
constexpr int kMaxChunksPerWave = 4;          // 4 KiB of K or of V in flight per wave

// ---------------------------------------------------------------------------
// Device error flag (replaces the page's device assert on a bad slot id).
// One 64-bit word per device: bits 0-31 hold the smallest rejected token
// (0xFFFFFFFF if none; token positions stay below 2^32 - 1), bits 32-63 the
// number of rejected tokens, saturating at 2^32 - 1.  Every report is one
// compare-and-swap and every take one exchange, so a take always sees the
// count and the smallest token of the same set of reports.
// ---------------------------------------------------------------------------
constexpr unsigned long long kFlagClear = 0xFFFFFFFFull;
__device__ unsigned long long g_kvstore_error = kFlagClear;

__device__ __forceinline__ unsigned long long flag_with(unsigned long long f, uint32_t token) {
  const uint32_t first = (uint32_t)f < token ? (uint32_t)f : token;
  const uint32_t count = (uint32_t)(f >> 32);
  return ((unsigned long long)(count == 0xFFFFFFFFu ? count : count + 1u) << 32) | first;
}

__device__ __forceinline__ void report_bad_token(uint32_t token) {
  unsigned long long seen = kFlagClear;
  for (;;) {
    const unsigned long long prev = atomicCAS(&g_kvstore_error, seen, flag_with(seen, token));
    if (prev == seen) return;
    seen = prev;
  }
}

// Takes the flag into out[0] (smallest bad token, or -1) and out[1] (count),
// leaving it cleared.  One thread.
__global__ void kvstore_take_error_kernel(int64_t* out) {
  const unsigned long long f = atomicExch(&g_kvstore_error, kFlagClear);
  const uint32_t count = (uint32_t)(f >> 32);
  out[0] = count ? (int64_t)(uint32_t)f : -1;
  out[1] = (int64_t)count;
}

// Where kvstore_check_error takes the flag to, per device; one check at a time.
__device__ int64_t g_kvstore_taken[2];

__device__ __forceinline__ uint32_t wave_uniform(uint32_t x) {
  return __builtin_amdgcn_readfirstlane(x);
}

template <typename IdxT>
__device__ __forceinline__ int64_t load_index(const void* indices, int64_t pos) {
  return (int64_t)static_cast<const IdxT*>(indices)[pos];
}

// Marks a loaded value as needed at this point.  Placed after the last load
// of a wave, once per loaded value, it keeps every load of the wave ahead of
// the first wait for one: left alone, the compiler may sink a load into the
// (divergent) block of its store, widen an index where it is loaded, or move
// the wave's scalar index load behind a long computation on the row, and then
// waits for each load before it issues the next, one memory latency after
// another.  The value stays in its register; no instruction is emitted.
template <typename T>
__device__ __forceinline__ void loaded(T& v) { asm volatile("" : "+v"(v)); }

// The wave's index, loaded after the row loads are issued.  A scalar index
// load issued before them would be waited for together with the kernel
// arguments that the row addresses need (scalar loads return out of order,
// so a wave can only wait for all of them), delaying the row loads by the
// index latency.  The array address passes through a scalar register at this
// point, so the load cannot be moved above it; it is read as constant memory
// (the kernel never writes the index array), which keeps it a scalar load;
// and the value is asked for right here, before the row data, so that the
// load is not moved below the waits for the row either.
template <typename IdxT>
__device__ __forceinline__ __attribute__((address_space(4))) const IdxT* indices_after_row_loads(
    const void* indices) {
  uint64_t a = reinterpret_cast<uint64_t>(indices);
  asm volatile("" : "+s"(a));
  return reinterpret_cast<__attribute__((address_space(4))) const IdxT*>(a);
}
__device__ __forceinline__ void index_needed_here(int64_t& loc) { asm volatile("" : "+s"(loc)); }

template <typename IdxT>
__device__ __forceinline__ int64_t load_index_after_row_loads(const void* indices, int64_t pos) {
  int64_t loc = (int64_t)indices_after_row_loads<IdxT>(indices)[pos];
  index_needed_here(loc);
  return loc;
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Vector of VW bytes moved by one lane in one access (16, 8 or 4).
template <int VW> struct LaneVec;
template <> struct LaneVec<16> { typedef u32x4 type; };
template <> struct LaneVec<8> { typedef u32x2 type; };
template <> struct LaneVec<4> { typedef uint32_t type; };

template <int VW>
__device__ __forceinline__ typename LaneVec<VW>::type loadv(const uint8_t* base, uint32_t off) {
  typedef typename LaneVec<VW>::type T;
  return __builtin_nontemporal_load(reinterpret_cast<const T*>(base + off));
}

template <int VW>
__device__ __forceinline__ void storev(uint8_t* base, uint32_t off, typename LaneVec<VW>::type v) {
  typedef typename LaneVec<VW>::type T;
  __builtin_nontemporal_store(v, reinterpret_cast<T*>(base + off));
}

__device__ __forceinline__ u32x4 load16(const uint8_t* base, uint32_t off) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + off));
}

// Raw buffer descriptor over [row, row + 2^31): stride 0, CDNA data format word.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(uint8_t* row) {
  return __builtin_amdgcn_make_buffer_rsrc(row, 0, 0x7FFFFFFF, 0x00020000);
}

// ---------------------------------------------------------------------------
// Scatter copy.
// ---------------------------------------------------------------------------
struct CopyParams {
  const uint8_t* k;
  const uint8_t* v;
  uint8_t* k_cache;
  uint8_t* v_cache;
  const void* indices;
  int64_t idx_stride;
  int64_t k_stride;
  int64_t v_stride;
  int64_t cache_stride;
  int64_t size_limit;
  uint32_t row_bytes;
  uint32_t batch;       // tokens of this launch
  uint32_t token_base;  // first token of this launch
};

// One row slice of K or of V of kTok consecutive tokens per wave.  Grid:
// x = ceil(batch / (kCopyWavesPerBlock * kTok)) blocks of kCopyWavesPerBlock
// waves; y = slices of the row, kChunks chunks of 64 * VW bytes each; z = 2:
// K (0) or V (1).  Blocks are dispatched x first, so a launch moves its K
// rows, then its V rows; K and V in separate waves of half the bytes let the
// residency cap be set in finer steps (2 KiB-row copy: 12 waves of 2 KiB per
// CU, 1.5% faster than the best cap of waves moving 2 KiB of K and 2 KiB of V
// each).  Several tokens per wave pay off for launches of few waves, where
// the dispatch of waves and the load-to-store turnaround of each wave weigh
// more than the bytes.
template <int VW, int kChunks, int kTok, typename IdxT>
__global__ __launch_bounds__(kCopyBlockThreads) void kvstore_copy_kernel(const CopyParams p) {
  typedef typename LaneVec<VW>::type T;
  constexpr uint32_t kChunk = kWave * VW;
  const uint32_t lane = threadIdx.x % kWave;
  // A wave past the batch (in the last block) does not return at once: it
  // loads the last token and stores nothing, so that no branch precedes the
  // loads and the kernel arguments arrive in one batch of scalar loads, not
  // two (same process: prefill copy 48.59-48.64 -> 48.42-48.46 us, wide
  // strided copy 7.76-7.81 -> 7.52-7.54).
  const uint32_t i0 = wave_uniform((blockIdx.x * kCopyWavesPerBlock + threadIdx.x / kWave) * kTok);
  const uint32_t slice = blockIdx.y;
  const bool is_v = blockIdx.z != 0;
  const uint8_t* base = is_v ? p.v : p.k;
  const int64_t stride = is_v ? p.v_stride : p.k_stride;
  const uint32_t col0 = slice * (kChunks * kChunk) + lane * VW;

  // Lanes past the row load the row's last VW bytes, tokens past the batch
  // load the last token, and neither stores: no load sits under a branch.
  T r[kTok][kChunks];
#pragma unroll
  for (int t = 0; t < kTok; ++t) {
    const uint32_t it = i0 + t < p.batch ? i0 + t : p.batch - 1;
    const uint8_t* src = base + (int64_t)(p.token_base + it) * stride;
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const uint32_t col = col0 + c * kChunk;
      r[t][c] = loadv<VW>(src, col < p.row_bytes ? col : p.row_bytes - VW);
    }
  }
  const auto idx = indices_after_row_loads<IdxT>(p.indices);
  int64_t loc[kTok];
#pragma unroll
  for (int t = 0; t < kTok; ++t) {
    const uint32_t it = i0 + t < p.batch ? i0 + t : p.batch - 1;
    loc[t] = (int64_t)idx[(int64_t)(p.token_base + it) * p.idx_stride];
  }
#pragma unroll
  for (int t = 0; t < kTok; ++t) index_needed_here(loc[t]);
#pragma unroll
  for (int t = 0; t < kTok; ++t)
#pragma unroll
    for (int c = 0; c < kChunks; ++c) loaded(r[t][c]);

  uint8_t* const cache = is_v ? p.v_cache : p.k_cache;
#pragma unroll
  for (int t = 0; t < kTok; ++t) {
    if (i0 + t >= p.batch) break;
    if (loc[t] < 0 || loc[t] >= p.size_limit) {
      if (lane == 0 && slice == 0 && !is_v) report_bad_token(p.token_base + i0 + t);
      continue;
    }
    uint8_t* dst = cache + loc[t] * p.cache_stride;
    // Non-temporal stores: sc1 stores timed 48.0 against 48.6 us for the
    // prefill copy alone, but left written lines for the next kernel to
    // write back (copy then fused FP8 store, alternating: 68.4 against 66.1
    // us per pair).
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const uint32_t col = col0 + c * kChunk;
      if (col < p.row_bytes) storev<VW>(dst, col, r[t][c]);
    }
  }
}

// Several rows per wave, for rows that need at most 32 lanes.  Each aligned
// group of 2^group_shift lanes owns kPackRows tokens (indices are per-lane
// loads); lane c of a group moves bytes [c * VW, c * VW + VW) of each row.
// Every lane loads (past the batch the last token, past the row the row's
// last VW bytes) and only lanes inside both store, so all loads of a wave are
// issued before its first wait.  Blocks of kPackWavesPerBlock waves; grid
// x = ceil(batch / tokens per block).  256 B rows of the 32768-token
// tensor-parallel share: 4 tokens per group (16 per wave) 6.72 us, 2 tokens
// 8.1, 8 tokens 7.0, 16 tokens 7.3-8.0.
constexpr int kPackWavesPerBlock = 4;
constexpr int kPackRows = 4;

template <int VW, typename IdxT>
__global__ __launch_bounds__(kWave * kPackWavesPerBlock) void kvstore_copy_packed_kernel(
    const CopyParams p, uint32_t group_shift) {
  typedef typename LaneVec<VW>::type T;
  const uint32_t lane = threadIdx.x % kWave;
  const uint32_t wave = blockIdx.x * kPackWavesPerBlock + threadIdx.x / kWave;
  const uint32_t rows_per_wave = kWave >> group_shift;
  const uint32_t col = (lane & ((1u << group_shift) - 1)) * VW;
  const bool active = col < p.row_bytes;
  const uint32_t lcol = active ? col : p.row_bytes - VW;
  T kr[kPackRows], vr[kPackRows];
  IdxT idx[kPackRows];
#pragma unroll
  for (int r = 0; r < kPackRows; ++r) {
    const uint64_t i = ((uint64_t)wave * kPackRows + r) * rows_per_wave + (lane >> group_shift);
    const int64_t t = (int64_t)p.token_base + (int64_t)(i < p.batch ? i : p.batch - 1);
    idx[r] = static_cast<const IdxT*>(p.indices)[t * p.idx_stride];
    kr[r] = loadv<VW>(p.k + t * p.k_stride, lcol);
    vr[r] = loadv<VW>(p.v + t * p.v_stride, lcol);
  }
#pragma unroll
  for (int r = 0; r < kPackRows; ++r) {
    loaded(idx[r]);
    loaded(kr[r]);
    loaded(vr[r]);
  }
#pragma unroll
  for (int r = 0; r < kPackRows; ++r) {
    const uint64_t i = ((uint64_t)wave * kPackRows + r) * rows_per_wave + (lane >> group_shift);
    if (i >= p.batch) continue;
    const int64_t loc = (int64_t)idx[r];
    if (loc < 0 || loc >= p.size_limit) {
      if (col == 0) report_bad_token(p.token_base + (uint32_t)i);
      continue;
    }
    if (active) {
      storev<VW>(p.k_cache + loc * p.cache_stride, col, kr[r]);
      storev<VW>(p.v_cache + loc * p.cache_stride, col, vr[r]);
    }
  }
}

// ---------------------------------------------------------------------------
// Fused e4m3fn quantise + paged store.
// ---------------------------------------------------------------------------
struct Fp8Params {
  const uint8_t* k;
  const uint8_t* v;
  uint8_t* k_cache;
  uint8_t* v_cache;
  const void* indices;
  const float* inv_k;
  const float* inv_v;
  int64_t idx_stride;
  int64_t k_stride_token, k_stride_head;
  int64_t v_stride_token, v_stride_head;
  int64_t kc_stride_page, kc_stride_offset, kc_stride_head;
  int64_t vc_stride_page, vc_stride_offset, vc_stride_head;
  int64_t size_limit;
  int64_t page_size;
  uint32_t batch;           // tokens of this launch
  uint32_t token_base;      // first token of this launch
  uint32_t units;           // 16-element units per row: num_heads * head_dim / 16
  uint32_t units_per_head;  // head_dim / 16
  int32_t page_shift;       // log2(page_size) when a power of two, else -1
  int32_t linear_pages;     // both caches have page stride == page_size * offset stride
};

// Exact widening of the two bf16 values packed in a 32-bit word.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// Largest finite magnitude of the FP8 storage format: e4m3fn 448, e5m2 57344.
template <bool kE5M2>
__device__ __forceinline__ constexpr float fp8_max() {
  return kE5M2 ? 57344.0f : 448.0f;
}

// fp32 product, then clamp to the largest finite magnitude.  A NaN input is
// its own product (keeping its sign, whichever operand the multiply would
// return); a NaN fails the comparison and passes through; infinities clamp.
template <bool kE5M2>
__device__ __forceinline__ float scale_sat(float x, float inv) {
  const float y = (x != x) ? x : __fmul_rn(x, inv);
  return (__builtin_fabsf(y) > fp8_max<kE5M2>()) ? __builtin_copysignf(fp8_max<kE5M2>(), y) : y;
}

// Sign bits of four fp32 values, one per byte (bit 7 of byte i = sign of i).
__device__ __forceinline__ uint32_t sign_bytes(float a, float b, float c, float d) {
  return (__float_as_uint(a) >> 24) | ((__float_as_uint(b) >> 16) & 0xFF00u) |
         ((__float_as_uint(c) >> 8) & 0xFF0000u) | (__float_as_uint(d) & 0xFF000000u);
}

// Hardware round-to-nearest-even packed conversion of two fp32 values into
// the low (hi = false) or high half of a word.
template <bool kE5M2>
__device__ __forceinline__ int cvt_pk(float a, float b, int old, bool hi) {
  if constexpr (kE5M2)
    return hi ? __builtin_amdgcn_cvt_pk_bf8_f32(a, b, old, true)
              : __builtin_amdgcn_cvt_pk_bf8_f32(a, b, old, false);
  else
    return hi ? __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, true)
              : __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, false);
}

// Four saturated fp32 values -> four FP8 bytes (a first in the low byte).
// The inputs are already clamped to the largest finite magnitude, so a byte
// whose magnitude bits exceed the largest finite code (e4m3fn 0x7E, e5m2
// 0x7B) can only come from a NaN; the converter's NaN code is replaced by
// 0x7F | sign (the gfx950 converter writes every e4m3fn NaN as 0xFF).
template <bool kE5M2>
__device__ __forceinline__ uint32_t pack_fp8(float a, float b, float c, float d) {
  int w = cvt_pk<kE5M2>(a, b, 0, false);
  w = cvt_pk<kE5M2>(c, d, w, true);
  uint32_t u = (uint32_t)w;
  // 0x80 in each byte whose low seven bits exceed the largest finite code:
  // adding (0x7F - max) carries into bit 7 exactly then, never into the next byte.
  constexpr uint32_t bump = kE5M2 ? 0x04040404u : 0x01010101u;
  const uint32_t nan = ((u & 0x7F7F7F7Fu) + bump) & 0x80808080u;
  if (nan) {
    const uint32_t bytes = (nan >> 7) * 0xFFu;
    const uint32_t code = (0x7F7F7F7Fu | (sign_bytes(a, b, c, d) & 0x80808080u)) & bytes;
    u = (u & ~bytes) | code;
  }
  return u;
}

// 16 source elements (two 16-byte vectors) -> 16 FP8 bytes: the 8 elements
// of a scaled by inv_a give bytes 0-7, the 8 of b scaled by inv_b bytes 8-15.
// The exact path: clamp with NaN passed through, then the NaN code fix-up.
template <bool kFp16, bool kE5M2>
__device__ __forceinline__ u32x4 quantize16(u32x4 a, u32x4 b, float inv_a, float inv_b) {
  u32x4 out;
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w0 = w[2 * i], w1 = w[2 * i + 1];
    const float inv = i < 2 ? inv_a : inv_b;
    float e0, e1, e2, e3;
    if constexpr (kFp16) {
      e0 = f16_lo(w0); e1 = f16_hi(w0); e2 = f16_lo(w1); e3 = f16_hi(w1);
    } else {
      e0 = bf16_lo(w0); e1 = bf16_hi(w0); e2 = bf16_lo(w1); e3 = bf16_hi(w1);
    }
    out[i] = pack_fp8<kE5M2>(scale_sat<kE5M2>(e0, inv), scale_sat<kE5M2>(e1, inv),
                             scale_sat<kE5M2>(e2, inv), scale_sat<kE5M2>(e3, inv));
  }
  return out;
}

// 16 source elements -> 16 FP8 bytes with no clamp before the conversion.
// Where no byte comes out as a NaN or infinity code this equals quantize16:
// a product between the largest finite value and half a step above it
// rounds down to that value anyway.  A NaN product, or one further out,
// gives such a code (gfx950 converts them to NaN, e5m2 also to infinity).
template <bool kFp16, bool kE5M2>
__device__ __forceinline__ u32x4 quantize16_unclamped(u32x4 a, u32x4 b, float inv_a, float inv_b) {
  u32x4 out;
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w0 = w[2 * i], w1 = w[2 * i + 1];
    const float inv = i < 2 ? inv_a : inv_b;
    float e0, e1, e2, e3;
    if constexpr (kFp16) {
      e0 = f16_lo(w0); e1 = f16_hi(w0); e2 = f16_lo(w1); e3 = f16_hi(w1);
    } else {
      e0 = bf16_lo(w0); e1 = bf16_hi(w0); e2 = bf16_lo(w1); e3 = bf16_hi(w1);
    }
    int q = cvt_pk<kE5M2>(__fmul_rn(e0, inv), __fmul_rn(e1, inv), 0, false);
    q = cvt_pk<kE5M2>(__fmul_rn(e2, inv), __fmul_rn(e3, inv), q, true);
    out[i] = (uint32_t)q;
  }
  return out;
}

// True if a byte of q has magnitude bits above the largest finite code
// (e4m3fn 0x7E, e5m2 0x7B): a NaN or infinity code.
template <bool kE5M2>
__device__ __forceinline__ bool any_special(u32x4 q) {
  constexpr uint32_t bump = kE5M2 ? 0x04040404u : 0x01010101u;
  const uint32_t acc = ((q.x & 0x7F7F7F7Fu) + bump) | ((q.y & 0x7F7F7F7Fu) + bump) |
                       ((q.z & 0x7F7F7F7Fu) + bump) | ((q.w & 0x7F7F7F7Fu) + bump);
  return (acc & 0x80808080u) != 0;
}

// quantize16 for any inputs and scales: the unclamped conversion, and the
// exact path for the lanes it leaves with a NaN or infinity code, behind a
// wave-uniform branch (not taken unless some lane needs it).
template <bool kFp16, bool kE5M2>
__device__ __forceinline__ u32x4 quantize16_checked(u32x4 a, u32x4 b, float inv_a, float inv_b) {
  u32x4 q = quantize16_unclamped<kFp16, kE5M2>(a, b, inv_a, inv_b);
  const bool special = any_special<kE5M2>(q);
  if (__builtin_expect(__ballot(special) != 0, 0)) {
    if (special) q = quantize16<kFp16, kE5M2>(a, b, inv_a, inv_b);
  }
  return q;
}

// Byte offsets of 8-element group g inside one token's source row (16 bytes
// per group) and inside one cache slot (8 bytes per group).  kFlat: heads are
// back to back in both (offsets linear in g).
template <bool kFlat>
__device__ __forceinline__ void group_offsets(uint32_t g, uint32_t groups_per_head,
                                              int64_t src_head, int64_t dst_head,
                                              uint32_t* src_off, uint32_t* dst_off) {
  if constexpr (kFlat) {
    *src_off = g * 16u;
    *dst_off = g * 8u;
  } else {
    const uint32_t h = g / groups_per_head;
    const uint32_t r = g - h * groups_per_head;
    *src_off = (uint32_t)(h * src_head) + r * 16u;
    *dst_off = (uint32_t)(h * dst_head) + r * 8u;
  }
}

// 8-byte store with the sc1 cache policy (bit 4 of the buffer cache-policy operand).
__device__ __forceinline__ void store8_sc1(__amdgpu_buffer_rsrc_t row, uint32_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, row, (int)off, 0, 16);
}

// One tensor (K or V) of one token, as the wave sees it.
struct TensorView {
  const uint8_t* src;   // this token's input row
  int64_t src_head;
  uint8_t* cache;
  int64_t c_page, c_offset, c_head;
  const float* inv;
};

__device__ __forceinline__ TensorView tensor_view(const Fp8Params& p, bool is_v, uint32_t token) {
  TensorView t;
  t.src = (is_v ? p.v : p.k) + (int64_t)token * (is_v ? p.v_stride_token : p.k_stride_token);
  t.src_head = is_v ? p.v_stride_head : p.k_stride_head;
  t.cache = is_v ? p.v_cache : p.k_cache;
  t.c_page = is_v ? p.vc_stride_page : p.kc_stride_page;
  t.c_offset = is_v ? p.vc_stride_offset : p.kc_stride_offset;
  t.c_head = is_v ? p.vc_stride_head : p.kc_stride_head;
  t.inv = is_v ? p.inv_v : p.inv_k;
  return t;
}

// Byte offset of slot loc in a paged cache with the given page/offset strides.
__device__ __forceinline__ int64_t slot_offset(const Fp8Params& p, int64_t loc, int64_t c_page,
                                               int64_t c_offset) {
  if (p.linear_pages) return loc * c_offset;
  int64_t page, off;
  if (p.page_shift >= 0) {
    page = loc >> p.page_shift;
    off = loc & (p.page_size - 1);
  } else {
    page = loc / p.page_size;
    off = loc - page * p.page_size;
  }
  return page * c_page + off * c_offset;
}

// How the FP8 stores load their rows.  Loads under a branch per group (zeros
// past the row) suit one pass and bf16 rows of several passes: the compiler
// keeps every load ahead of the first wait.  For fp16 rows of several passes
// it issues only the first two loads before waiting on them, one memory
// latency after another, so there every lane loads (a group past the row
// reads the row's last group and stores nothing) and the values are pinned
// after the last load.  16384 tokens of 16x128 fp16: static store 37.41 ->
// 37.07 us, per-token scales 39.74 -> 38.78; 8192 tokens of 32x128 fp16 with
// per-token-head scales 44.95 -> 41.11.  The same form measured 0.9 us
// slower for 16x128 bf16 rows and 0.3 us slower for one pass.
template <int kPasses, bool kFp16>
constexpr bool kUnconditionalLoads = kPasses > 1 && kFp16;

// Grid: x = ceil(batch / kWavesPerBlock), one wave per token; y = 2 * slices:
// bit 0 selects K (0) or V (1), the rest the slice of kPasses * 64 units.
// K and V of a token go to separate waves: twice the waves of half the size
// measured ~7% faster than one wave doing both.
template <int kPasses, bool kFlat, bool kFp16, bool kE5M2, typename IdxT>
__global__ __launch_bounds__(kBlockThreads) void kvstore_fp8_paged_kernel(const Fp8Params p) {
  const uint32_t lane = threadIdx.x % kWave;
  // A wave past the batch loads the last token and returns before storing,
  // so that no branch precedes the loads (the kernel arguments then arrive in
  // one batch of scalar loads: 17.34 -> 17.17 us on the 16384-token workload).
  const uint32_t i = wave_uniform(blockIdx.x * kWavesPerBlock + threadIdx.x / kWave);
  const bool valid = i < p.batch;
  const uint32_t token = p.token_base + (valid ? i : p.batch - 1);
  const bool is_v = (blockIdx.y & 1u) != 0;
  const uint32_t slice = blockIdx.y >> 1;

  const int64_t loc = load_index<IdxT>(p.indices, (int64_t)token * p.idx_stride);
  const TensorView t = tensor_view(p, is_v, token);
  const float inv = t.inv ? *t.inv : 1.0f;

  // Each pass covers 128 groups of 8 elements (1024 elements): lane l takes
  // groups l and l + 64, so each load instruction of the wave reads 1 KiB of
  // consecutive groups and each store writes 512 bytes of them.
  const uint32_t groups = 2u * p.units;
  const uint32_t groups_per_head = 2u * p.units_per_head;
  u32x4 a[kPasses], b[kPasses];
  uint32_t da[kPasses], db[kPasses];
  if constexpr (kUnconditionalLoads<kPasses, kFp16>) {
#pragma unroll
    for (int i = 0; i < kPasses; ++i) {
      const uint32_t g = (slice * kPasses + i) * (2u * kWave) + lane;
      uint32_t so;
      group_offsets<kFlat>(g < groups ? g : groups - 1, groups_per_head, t.src_head, t.c_head, &so,
                           &da[i]);
      a[i] = load16(t.src, so);
      group_offsets<kFlat>(g + kWave < groups ? g + kWave : groups - 1, groups_per_head,
                           t.src_head, t.c_head, &so, &db[i]);
      b[i] = load16(t.src, so);
    }
#pragma unroll
    for (int i = 0; i < kPasses; ++i) {
      loaded(a[i]);
      loaded(b[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < kPasses; ++i) {
      const uint32_t g = (slice * kPasses + i) * (2u * kWave) + lane;
      a[i] = u32x4{0u, 0u, 0u, 0u};
      b[i] = u32x4{0u, 0u, 0u, 0u};
      uint32_t so;
      if (g < groups) {
        group_offsets<kFlat>(g, groups_per_head, t.src_head, t.c_head, &so, &da[i]);
        a[i] = load16(t.src, so);
      }
      if (g + kWave < groups) {
        group_offsets<kFlat>(g + kWave, groups_per_head, t.src_head, t.c_head, &so, &db[i]);
        b[i] = load16(t.src, so);
      }
    }
  }

  if (!valid) return;
  if (loc < 0 || loc >= p.size_limit) {
    if (lane == 0 && slice == 0 && !is_v) report_bad_token(token);
    return;
  }
  const __amdgpu_buffer_rsrc_t d = row_rsrc(t.cache + slot_offset(p, loc, t.c_page, t.c_offset));
#pragma unroll
  for (int i = 0; i < kPasses; ++i) {
    const uint32_t g = (slice * kPasses + i) * (2u * kWave) + lane;
    if (g < groups) {
      // bytes 0-7 of q come from group g (a), bytes 8-15 from group g + 64 (b)
      const u32x4 q = quantize16_checked<kFp16, kE5M2>(a[i], b[i], inv, inv);
      store8_sc1(d, da[i], u32x2{q.x, q.y});
      if (g + kWave < groups) store8_sc1(d, db[i], u32x2{q.z, q.w});
    }
  }
}

// ---------------------------------------------------------------------------
// Fused e4m3fn quantise + paged store with dynamic scales.
// ---------------------------------------------------------------------------
constexpr int kMaxDynPasses = 4;   // whole row in one wave: up to 4096 elements
constexpr int kMaxDynHeads = kMaxDynPasses * 1024 / 16;  // heads of at least 16 elements

struct Fp8DynParams {
  Fp8Params base;                  // inv_k / inv_v unused
  uint8_t* k_scales;
  uint8_t* v_scales;
  int64_t ks_stride_page, ks_stride_offset, ks_stride_head;
  int64_t vs_stride_page, vs_stride_offset, vs_stride_head;
};

// max |x| over the 8 source elements of one 16-byte vector; NaN elements are
// ignored (fmaxf), so the result is a non-negative float that is never NaN.
template <bool kFp16>
__device__ __forceinline__ float amax8(u32x4 a) {
  const uint32_t w[4] = {a.x, a.y, a.z, a.w};
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float lo, hi;
    if constexpr (kFp16) {
      lo = f16_lo(w[i]); hi = f16_hi(w[i]);
    } else {
      lo = bf16_lo(w[i]); hi = bf16_hi(w[i]);
    }
    m = __builtin_fmaxf(m, __builtin_fmaxf(__builtin_fabsf(lo), __builtin_fabsf(hi)));
  }
  return m;
}

// A magnitude |x| of a bf16 / fp16 element as its 15-bit pattern (sign
// cleared), and back.  For values that are not NaN these patterns order like
// the magnitudes, and the conversions are exact.
template <bool kFp16>
__device__ __forceinline__ float mag_to_float(uint32_t m) {
  if constexpr (kFp16) return (float)__builtin_bit_cast(_Float16, (uint16_t)m);
  else return __uint_as_float(m << 16);
}
template <bool kFp16>
__device__ __forceinline__ uint32_t float_to_mag(float f) {
  if constexpr (kFp16) return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
  else return __float_as_uint(f) >> 16;
}

// max |x| over the 8 elements of one 16-byte vector, as a magnitude pattern:
// the patterns compared directly, two per packed 16-bit max.  Exact when no
// element is NaN (a NaN pattern would win; such lanes take amax8 instead).
__device__ __forceinline__ uint32_t amax8_mag(u32x4 a) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  const u16x2 m = __builtin_elementwise_max(
      __builtin_elementwise_max(__builtin_bit_cast(u16x2, a.x & 0x7FFF7FFFu),
                                __builtin_bit_cast(u16x2, a.y & 0x7FFF7FFFu)),
      __builtin_elementwise_max(__builtin_bit_cast(u16x2, a.z & 0x7FFF7FFFu),
                                __builtin_bit_cast(u16x2, a.w & 0x7FFF7FFFu)));
  return m.x > m.y ? m.x : m.y;
}

// One DPP step of a lane max: each lane takes the larger of its value and the
// value of the lane that the row permutation kCtrl selects.
template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_max(uint32_t v) {
  const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kCtrl, 0xF, 0xF, false);
  return v > o ? v : o;
}

// Unsigned max over aligned groups of `lanes` lanes (a power of two <= 64).
// Groups of up to 16 lanes reduce inside a DPP row (quad swaps, then the
// half-row and row mirrors); a 32-lane group adds one cross-row shuffle, and
// the whole wave combines its four rows with readlane.
__device__ __forceinline__ uint32_t group_max(uint32_t v, uint32_t lanes) {
  if (lanes >= 2) v = dpp_max<0xB1>(v);    // quad_perm [1,0,3,2]: lane ^ 1
  if (lanes >= 4) v = dpp_max<0x4E>(v);    // quad_perm [2,3,0,1]: lane ^ 2
  if (lanes >= 8) v = dpp_max<0x141>(v);   // row_half_mirror: the other quad of 8
  if (lanes >= 16) v = dpp_max<0x140>(v);  // row_mirror: the other 8 of the row
  if (lanes == 64) {
    const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
    const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
    const uint32_t lo = r0 > r1 ? r0 : r1, hi = r2 > r3 ? r2 : r3;
    v = lo > hi ? lo : hi;
  } else if (lanes == 32) {
    const uint32_t o = (uint32_t)__shfl_xor((int)v, 16);
    v = v > o ? v : o;
  }
  return v;
}

// fp32 scale of a group, at least the smallest normal float.
__device__ __forceinline__ float dyn_scale(float amax) {
  return __builtin_fmaxf(amax / 448.0f, 1.17549435e-38f);
}

// Grid: x = ceil(batch / kDynWavesPerBlock), one wave per token; y = 2: K (0) or
// V (1).  The wave holds the tensor's whole row: kPasses passes of 1024
// elements, as in the static store (lane l takes 8-element groups l and
// l + 64 of each pass).  kPerHead false: one scale covers the row.  Per head,
// with gph = head_dim / 8 groups per head: for gph <= 64 each head lies
// wholly in the first or the second group of its lanes, on gph aligned lanes;
// for gph = 128 (head_dim 1024) a head is one whole pass.  Group maxima are
// taken on the 15-bit magnitude patterns of the 16-bit inputs and converted
// to fp32 once per group.
template <int kPasses, bool kFlat, bool kFp16, bool kPerHead, typename IdxT>
__global__ __launch_bounds__(kWave * kDynWavesPerBlock) void kvstore_fp8_dynamic_kernel(const Fp8DynParams d) {
  const Fp8Params& p = d.base;
  const uint32_t lane = threadIdx.x % kWave;
  const uint32_t w = threadIdx.x / kWave;
  const uint32_t i = wave_uniform(blockIdx.x * kDynWavesPerBlock + w);
  // The waves of a block meet at a barrier before the scale store, so a wave
  // past the batch works on the last token and stores nothing.
  const bool valid = i < p.batch;
  const uint32_t token = p.token_base + (valid ? i : p.batch - 1);
  const bool is_v = blockIdx.y != 0;

  const int64_t loc = load_index<IdxT>(p.indices, (int64_t)token * p.idx_stride);
  const TensorView t = tensor_view(p, is_v, token);
  const uint32_t groups = 2u * p.units;
  const uint32_t gph = 2u * p.units_per_head;

  u32x4 a[kPasses], b[kPasses];
  uint32_t da[kPasses], db[kPasses];
  if constexpr (kUnconditionalLoads<kPasses, kFp16>) {
#pragma unroll
    for (int j = 0; j < kPasses; ++j) {
      const uint32_t g = j * (2u * kWave) + lane;
      uint32_t so;
      group_offsets<kFlat>(g < groups ? g : groups - 1, gph, t.src_head, t.c_head, &so, &da[j]);
      a[j] = load16(t.src, so);
      group_offsets<kFlat>(g + kWave < groups ? g + kWave : groups - 1, gph, t.src_head, t.c_head,
                           &so, &db[j]);
      b[j] = load16(t.src, so);
    }
#pragma unroll
    for (int j = 0; j < kPasses; ++j) {
      loaded(a[j]);
      loaded(b[j]);
    }
    // groups past the row take no part in the maxima
#pragma unroll
    for (int j = 0; j < kPasses; ++j) {
      const uint32_t g = j * (2u * kWave) + lane;
      if (g >= groups) a[j] = u32x4{0u, 0u, 0u, 0u};
      if (g + kWave >= groups) b[j] = u32x4{0u, 0u, 0u, 0u};
    }
  } else {
#pragma unroll
    for (int j = 0; j < kPasses; ++j) {
      const uint32_t g = j * (2u * kWave) + lane;
      a[j] = u32x4{0u, 0u, 0u, 0u};
      b[j] = u32x4{0u, 0u, 0u, 0u};
      uint32_t so;
      if (g < groups) {
        group_offsets<kFlat>(g, gph, t.src_head, t.c_head, &so, &da[j]);
        a[j] = load16(t.src, so);
      }
      if (g + kWave < groups) {
        group_offsets<kFlat>(g + kWave, gph, t.src_head, t.c_head, &so, &db[j]);
        b[j] = load16(t.src, so);
      }
    }
  }
  // Every lane takes part in the lane reductions below (groups past the row
  // hold zeros), so the bounds check comes after them.
  // NaN patterns are the largest magnitude patterns, so a pass holds a NaN
  // exactly when its largest pattern lies above the infinity's.
  constexpr uint32_t kInfMag = kFp16 ? 0x7C00u : 0x7F80u;
  bool nan[kPasses];
  bool some_nan = false;
  uint32_t ma[kPasses], mb[kPasses];
#pragma unroll
  for (int j = 0; j < kPasses; ++j) {
    ma[j] = amax8_mag(a[j]);
    mb[j] = amax8_mag(b[j]);
    nan[j] = max(ma[j], mb[j]) > kInfMag;
    some_nan = some_nan || nan[j];
  }
  // Lanes holding a NaN take the maxima that ignore NaN elements, behind a
  // wave-uniform branch so that the common case does not compute them.
  if (__builtin_expect(__ballot(some_nan) != 0, 0)) {
#pragma unroll
    for (int j = 0; j < kPasses; ++j) {
      if (nan[j]) {
        ma[j] = float_to_mag<kFp16>(amax8<kFp16>(a[j]));
        mb[j] = float_to_mag<kFp16>(amax8<kFp16>(b[j]));
      }
    }
  }
  if constexpr (!kPerHead) {
    uint32_t mx = 0;
#pragma unroll
    for (int j = 0; j < kPasses; ++j) mx = max(mx, max(ma[j], mb[j]));
    mx = group_max(mx, kWave);
#pragma unroll
    for (int j = 0; j < kPasses; ++j) ma[j] = mb[j] = mx;
  } else if (gph > kWave) {
#pragma unroll
    for (int j = 0; j < kPasses; ++j) ma[j] = mb[j] = group_max(max(ma[j], mb[j]), kWave);
  } else {
#pragma unroll
    for (int j = 0; j < kPasses; ++j) {
      ma[j] = group_max(ma[j], gph);
      mb[j] = group_max(mb[j], gph);
    }
  }

  const bool in_range = loc >= 0 && loc < p.size_limit;
  // A rejected index addresses nothing: slot 0 stands in for it, so that no
  // offset below is formed from an arbitrary 64-bit value.
  const int64_t slot = in_range ? loc : 0;
  int64_t page, off;
  if (p.page_shift >= 0) {
    page = slot >> p.page_shift;
    off = slot & (p.page_size - 1);
  } else {
    page = slot / p.page_size;
    off = slot - page * p.page_size;
  }
  uint8_t* scales = is_v ? d.v_scales + page * d.vs_stride_page + off * d.vs_stride_offset
                         : d.k_scales + page * d.ks_stride_page + off * d.ks_stride_offset;
  const int64_t s_head = is_v ? d.vs_stride_head : d.ks_stride_head;
  // per-head scales need gph to be a power of two (checked on the host): the
  // head of group g is g >> log2(gph)
  const uint32_t gsh = __builtin_ctz(gph);
  float sa[kPasses], sb[kPasses];
#pragma unroll
  for (int j = 0; j < kPasses; ++j) {
    sa[j] = dyn_scale(mag_to_float<kFp16>(ma[j]));
    sb[j] = dyn_scale(mag_to_float<kFp16>(mb[j]));
  }

  // The scales of the block's waves (consecutive tokens) go through LDS to
  // wave 0, which stores them after the rows, behind a barrier that every
  // wave of the block reaches: where the tokens sit in consecutive slots the
  // scales leave as one memory request (per token-head, up to 64 of them per
  // instruction) instead of one or two per wave.  16384-token FP8 workload:
  // per token 17.97 us with blocks of four waves, 18.08 with two, 18.15 with
  // eight, 18.6-18.7 with a store per wave, and 17.84 against 17.99 with the
  // barrier after the row stores rather than before them; per token-head
  // 18.35-18.46 against 18.66-18.93 with two stores per wave.
  __shared__ float s_val[kDynWavesPerBlock][kPerHead ? kMaxDynHeads : 1];
  __shared__ float* s_at[kDynWavesPerBlock];
  if (lane == 0) s_at[w] = valid && in_range ? reinterpret_cast<float*>(scales) : nullptr;
  if constexpr (!kPerHead) {
    if (lane == 0) s_val[w][0] = sa[0];
  } else if ((lane & (gph - 1)) == 0) {
    // the first lane of each head's gph lanes, for the head of each of its
    // two groups (for gph = 128, lane 0: both groups lie in the pass's head)
#pragma unroll
    for (int j = 0; j < kPasses; ++j) {
      const uint32_t g = j * (2u * kWave) + lane;
      if (g < groups) s_val[w][g >> gsh] = sa[j];
      if (g + kWave < groups) s_val[w][(g + kWave) >> gsh] = sb[j];
    }
  }
  if (valid && !in_range && lane == 0 && !is_v) report_bad_token(token);
  if (valid && in_range) {
    const __amdgpu_buffer_rsrc_t dst = row_rsrc(t.cache + page * t.c_page + off * t.c_offset);
#pragma unroll
    for (int j = 0; j < kPasses; ++j) {
      const uint32_t g = j * (2u * kWave) + lane;
      if (g >= groups) continue;
      const bool has_b = g + kWave < groups;
      const float ia = 1.0f / sa[j], ib = 1.0f / sb[j];
      const u32x4 q = quantize16_checked<kFp16, false>(a[j], b[j], ia, ib);
      store8_sc1(dst, da[j], u32x2{q.x, q.y});
      if (has_b) store8_sc1(dst, db[j], u32x2{q.z, q.w});
    }
  }
  __syncthreads();
  if (w != 0) return;
  if constexpr (!kPerHead) {
    if (lane < (uint32_t)kDynWavesPerBlock && s_at[lane] != nullptr) *s_at[lane] = s_val[lane][0];
  } else {
    // lane e takes head e % heads of wave e / heads; per-head scale stores are
    // non-temporal (18.55-18.61 against 18.68-18.97 us with default-policy
    // stores, one store per head group)
    const uint32_t heads = groups >> gsh;
    for (uint32_t e = lane; e < (uint32_t)kDynWavesPerBlock * heads; e += kWave) {
      const uint32_t wv = e / heads, h = e - wv * heads;
      uint8_t* const at = reinterpret_cast<uint8_t*>(s_at[wv]);
      if (at != nullptr)
        __builtin_nontemporal_store(s_val[wv][h], reinterpret_cast<float*>(at + h * s_head));
    }
  }
}

// ---------------------------------------------------------------------------
// Host side: validation, dispatch, launch.
// ---------------------------------------------------------------------------
inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }
inline bool aligned(int64_t s, int64_t a) { return (s % a) == 0; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

constexpr int64_t kMaxGridY = 65535;

template <typename T> struct NoDeduce { typedef T type; };

// Launches `kernel` through hipLaunchKernel and returns that launch's own
// status, so an error left behind by an earlier, unrelated HIP call is
// neither reported as ours nor cleared.  KVSTORE_ERR_HIP means the runtime
// refused the launch (nothing ran).
template <typename... Args>
int launch(void (*kernel)(Args...), dim3 grid, dim3 block, uint32_t lds_bytes,
           hipStream_t stream, typename NoDeduce<Args>::type... args) {
  void* argv[] = {static_cast<void*>(&args)...};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, lds_bytes,
                         stream) == hipSuccess
             ? KVSTORE_OK
             : KVSTORE_ERR_HIP;
}

// Resident copy waves per CU, 0 for no cap.  Waves that load 2 KiB or more
// are capped to about 24 KiB of loads in flight per CU (2 KiB: 12 waves; at
// least 8): the copy writes rows at scattered slots, and the 2 KiB-row
// prefill copy measured 48.6 us at 12 resident waves against 49.1 at 10,
// 49.3 at 14, 49.4 at 16, 55 at 8 and 51.2 uncapped.  Smaller waves run
// uncapped: the 1152-byte rows of the wide strided copy measured 9.47 us
// uncapped, 9.49 at 22 waves and 9.9 at 18.
constexpr int64_t kCopyLoadBytesPerCU = 24 * 1024;
inline int64_t copy_waves_per_cu(int64_t load_bytes_per_wave) {
  if (load_bytes_per_wave < 2048) return 0;
  const int64_t w = kCopyLoadBytesPerCU / load_bytes_per_wave;
  return w < 8 ? 8 : w;
}

// Tokens per copy wave, for rows of up to two chunks, from the row bytes a
// launch reads: between 6 and 48 MiB a wave moves 8 tokens (uncapped);
// otherwise 1 (over 48 MiB under the residency cap).  Measured with rows in
// 16-slot runs over random pages: 8192 tokens of 1 KiB 6.70 against 8.61
// us, 2048 tokens of 2 KiB 4.25 against 5.22, 12288 tokens of 2 KiB 18.8
// against 19.5, the 8192-token wide strided copy 7.86 against 9.51; 16384
// tokens of 2 KiB 26.0 against 25.6 and the 32768-token prefill copy 53.0
// against 48.6 (2 and 4 tokens fell in between; 16 spilled registers and
// ran 2-3x slower).  Below, too few waves are left to fill the chip: 2 KiB
// rows replayed from a graph, 256 tokens 3.37 against 2.30 us, 1024 tokens
// 3.86 against 3.37, 2048 tokens 4.23 against 5.19.
constexpr int64_t kCopySmallLaunchMinBytes = 6ll << 20;
constexpr int64_t kCopySmallLaunchBytes = 48ll << 20;
constexpr int kCopySmallLaunchTokens = 8;
inline int copy_tokens_per_wave(int64_t read_bytes) {
  return read_bytes > kCopySmallLaunchMinBytes && read_bytes <= kCopySmallLaunchBytes
             ? kCopySmallLaunchTokens
             : 1;
}

// gfx950 allocates LDS to a block in units of 1280 bytes (a block asking for
// 23,405 bytes occupies 24,320: six such blocks fit in 160 KiB, not seven),
// so the size that lets n blocks share a CU is rounded down to that unit.
constexpr int64_t kLdsGranule = 1280;
inline uint32_t lds_for_blocks(int64_t lds_per_cu, int64_t blocks) {
  if (lds_per_cu <= 0 || blocks <= 0) return 0;
  return (uint32_t)(lds_per_cu / blocks / kLdsGranule * kLdsGranule);
}

// Tokens of one launch.  A grid with one wave per token then stays at 2^30
// work-items, well inside the 2^32 limit of a dispatch dimension; larger
// batches run as several launches on the same stream, in token order.
constexpr uint32_t kMaxLaunchTokens = 1u << 24;

// Calls fn(params) once per run of at most kMaxLaunchTokens tokens of
// [0, batch), with token_base / count set to the run.  Stops at the first
// status other than KVSTORE_OK.
template <typename P, typename F>
int launch_in_runs(P& params, uint32_t& token_base, uint32_t& count, uint32_t batch, F&& fn) {
  for (uint32_t base = 0; base < batch;) {
    const uint32_t n = batch - base < kMaxLaunchTokens ? batch - base : kMaxLaunchTokens;
    token_base = base;
    count = n;
    const int st = fn(static_cast<const P&>(params));
    if (st != KVSTORE_OK) return st;
    base += n;
  }
  return KVSTORE_OK;
}

// LDS bytes per CU of the current device (cached per device; calls from
// several threads may fill an entry concurrently with the same value), 0 if
// unknown.
int64_t lds_per_cu() {
  static std::atomic<int64_t> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int64_t have = cache[dev].load(std::memory_order_relaxed);
  if (have == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
            hipSuccess || v <= 0)
      return 0;
    have = v;
    cache[dev].store(have, std::memory_order_relaxed);
  }
  return have;
}

template <int VW, typename IdxT>
int launch_copy_vw(const CopyParams& p, hipStream_t stream) {
  constexpr int64_t kChunk = kWave * VW;
  const dim3 block(kCopyBlockThreads);
  const int64_t lanes = ceil_div(p.row_bytes, VW);
  if (lanes <= kWave / 2) {
    // several rows per wave: groups of the next power of two >= lanes
    uint32_t shift = 0;
    while ((int64_t(1) << shift) < lanes) ++shift;
    const int64_t rows_per_block = (int64_t)kPackWavesPerBlock * kPackRows * (kWave >> shift);
    const dim3 grid((uint32_t)ceil_div(p.batch, rows_per_block));
    return launch(kvstore_copy_packed_kernel<VW, IdxT>, grid, dim3(kWave * kPackWavesPerBlock), 0,
                  stream, p, shift);
  }
  const int64_t chunks = ceil_div(p.row_bytes, kChunk);
  const int per_wave = (int)(chunks < kMaxChunksPerWave ? chunks : kMaxChunksPerWave);
  const int64_t slices = ceil_div(chunks, per_wave);
  if (slices > kMaxGridY) return KVSTORE_ERR_SHAPE;
  const int tok = per_wave <= 2 ? copy_tokens_per_wave(2 * (int64_t)p.batch * p.row_bytes) : 1;
  const dim3 grid((uint32_t)ceil_div(p.batch, (int64_t)kCopyWavesPerBlock * tok), (uint32_t)slices, 2);
  // The kernel uses no LDS; the dynamic allocation only caps residency (tuned
  // for 16-byte lanes, where a wave has the most bytes in flight).
  const int64_t slice_bytes = (int64_t)per_wave * kChunk;
  const int64_t wave_bytes = p.row_bytes < slice_bytes ? (int64_t)p.row_bytes : slice_bytes;
  const int64_t waves_per_cu = VW == 16 && tok == 1 ? copy_waves_per_cu(wave_bytes) : 0;
  const uint32_t lds_bytes =
      waves_per_cu > 0 ? lds_for_blocks(lds_per_cu(), waves_per_cu / kCopyWavesPerBlock) : 0;
  constexpr int M = kCopySmallLaunchTokens;
  switch (per_wave * 16 + tok) {
    case 1 * 16 + 1: return launch(kvstore_copy_kernel<VW, 1, 1, IdxT>, grid, block, lds_bytes, stream, p);
    case 1 * 16 + M: return launch(kvstore_copy_kernel<VW, 1, M, IdxT>, grid, block, lds_bytes, stream, p);
    case 2 * 16 + 1: return launch(kvstore_copy_kernel<VW, 2, 1, IdxT>, grid, block, lds_bytes, stream, p);
    case 2 * 16 + M: return launch(kvstore_copy_kernel<VW, 2, M, IdxT>, grid, block, lds_bytes, stream, p);
    case 3 * 16 + 1: return launch(kvstore_copy_kernel<VW, 3, 1, IdxT>, grid, block, lds_bytes, stream, p);
    default: return launch(kvstore_copy_kernel<VW, 4, 1, IdxT>, grid, block, lds_bytes, stream, p);
  }
}

template <typename IdxT>
int launch_copy(const CopyParams& p, int vw, hipStream_t stream) {
  if (vw == 16) return launch_copy_vw<16, IdxT>(p, stream);
  if (vw == 8) return launch_copy_vw<8, IdxT>(p, stream);
  return launch_copy_vw<4, IdxT>(p, stream);
}

template <int kPasses, bool kFlat, bool kFp16, bool kE5M2>
int launch_fp8_idx(const Fp8Params& p, bool i64, dim3 grid, hipStream_t stream) {
  const dim3 block(kBlockThreads);
  if (i64)
    return launch(kvstore_fp8_paged_kernel<kPasses, kFlat, kFp16, kE5M2, int64_t>, grid, block, 0,
                  stream, p);
  return launch(kvstore_fp8_paged_kernel<kPasses, kFlat, kFp16, kE5M2, int32_t>, grid, block, 0,
                stream, p);
}

template <int kPasses, bool kE5M2>
int launch_fp8_fmt(const Fp8Params& p, bool flat, bool fp16, bool i64, dim3 grid,
                   hipStream_t stream) {
  if (flat)
    return fp16 ? launch_fp8_idx<kPasses, true, true, kE5M2>(p, i64, grid, stream)
                : launch_fp8_idx<kPasses, true, false, kE5M2>(p, i64, grid, stream);
  return fp16 ? launch_fp8_idx<kPasses, false, true, kE5M2>(p, i64, grid, stream)
              : launch_fp8_idx<kPasses, false, false, kE5M2>(p, i64, grid, stream);
}

template <int kPasses>
int launch_fp8_passes(const Fp8Params& p, bool flat, bool fp16, bool i64, bool e5m2, dim3 grid,
                      hipStream_t stream) {
  return e5m2 ? launch_fp8_fmt<kPasses, true>(p, flat, fp16, i64, grid, stream)
              : launch_fp8_fmt<kPasses, false>(p, flat, fp16, i64, grid, stream);
}

template <int kPasses, bool kFlat, bool kFp16, bool kPerHead>
int launch_dyn_idx(const Fp8DynParams& d, bool i64, dim3 grid, hipStream_t stream) {
  const dim3 block(kWave * kDynWavesPerBlock);
  if (i64)
    return launch(kvstore_fp8_dynamic_kernel<kPasses, kFlat, kFp16, kPerHead, int64_t>, grid,
                  block, 0, stream, d);
  return launch(kvstore_fp8_dynamic_kernel<kPasses, kFlat, kFp16, kPerHead, int32_t>, grid, block,
                0, stream, d);
}

template <int kPasses, bool kPerHead>
int launch_dyn_layout(const Fp8DynParams& d, bool flat, bool fp16, bool i64, dim3 grid,
                      hipStream_t stream) {
  if (flat)
    return fp16 ? launch_dyn_idx<kPasses, true, true, kPerHead>(d, i64, grid, stream)
                : launch_dyn_idx<kPasses, true, false, kPerHead>(d, i64, grid, stream);
  return fp16 ? launch_dyn_idx<kPasses, false, true, kPerHead>(d, i64, grid, stream)
              : launch_dyn_idx<kPasses, false, false, kPerHead>(d, i64, grid, stream);
}

template <int kPasses>
int launch_dyn_passes(const Fp8DynParams& d, bool per_head, bool flat, bool fp16, bool i64,
                      dim3 grid, hipStream_t stream) {
  return per_head ? launch_dyn_layout<kPasses, true>(d, flat, fp16, i64, grid, stream)
                  : launch_dyn_layout<kPasses, false>(d, flat, fp16, i64, grid, stream);
}

// Largest byte offset reached by [0, n) * stride must fit in int64 (stride >= 0).
bool fits(int64_t n, int64_t stride) {
  return stride == 0 || n <= INT64_MAX / stride;
}

// a + b + c <= INT64_MAX for non-negative a, b and c, without overflowing.
bool sum_fits(int64_t a, int64_t b, int64_t c) {
  return a <= INT64_MAX - b && a + b <= INT64_MAX - c;
}

// (n - 1) * stride + tail <= INT32_MAX, for n >= 1, stride >= 0 and
// 0 <= tail <= INT32_MAX, without overflowing: the last of n items at the
// given stride ends within 31 bits.
bool span_fits_int32(int64_t n, int64_t stride, int64_t tail) {
  if (tail > INT32_MAX) return false;
  return stride == 0 || n - 1 <= (INT32_MAX - tail) / stride;
}

// Index type, stride (>= 1, and batch * stride * 8 bytes addressable), alignment.
int check_index_args(const void* indices, int idx_dtype, int64_t idx_stride, uint32_t batch) {
  if (idx_dtype != KVSTORE_IDX_I32 && idx_dtype != KVSTORE_IDX_I64) return KVSTORE_ERR_DTYPE;
  if (idx_stride < 1 || idx_stride > INT64_MAX / 8 || !fits(batch, idx_stride * 8))
    return KVSTORE_ERR_SHAPE;
  if (!aligned(indices, idx_dtype == KVSTORE_IDX_I64 ? 8 : 4)) return KVSTORE_ERR_ALIGN;
  return KVSTORE_OK;
}

// Checks the arguments the two fused FP8 stores share and fills p (the scale
// pointers are left NULL).  Returns KVSTORE_OK or the status to return.
int fill_fp8_params(Fp8Params& p, const void* k, const void* v, void* k_cache, void* v_cache,
                    const void* indices, int idx_dtype, int64_t idx_stride, int32_t num_heads,
                    int32_t head_dim, int64_t k_stride_token_bytes, int64_t k_stride_head_bytes,
                    int64_t v_stride_token_bytes, int64_t v_stride_head_bytes,
                    int64_t kc_stride_page_bytes, int64_t kc_stride_offset_bytes,
                    int64_t kc_stride_head_bytes, int64_t vc_stride_page_bytes,
                    int64_t vc_stride_offset_bytes, int64_t vc_stride_head_bytes, uint32_t batch,
                    int64_t size_limit, int64_t page_size) {
  if (!k || !v || !k_cache || !v_cache || !indices) return KVSTORE_ERR_NULL;
  if (num_heads <= 0 || head_dim <= 0 || head_dim % 16) return KVSTORE_ERR_SHAPE;
  if (page_size <= 0 || size_limit <= 0) return KVSTORE_ERR_SHAPE;
  const int64_t strides[10] = {k_stride_token_bytes,   k_stride_head_bytes,
                               v_stride_token_bytes,   v_stride_head_bytes,
                               kc_stride_page_bytes,   kc_stride_offset_bytes,
                               kc_stride_head_bytes,   vc_stride_page_bytes,
                               vc_stride_offset_bytes, vc_stride_head_bytes};
  for (int64_t s : strides) {
    if (s < 0) return KVSTORE_ERR_SHAPE;
    if (!aligned(s, 16)) return KVSTORE_ERR_ALIGN;
  }
  // Per-lane offsets inside one token row / one slot are 32-bit.
  const int64_t heads = num_heads;
  if (!span_fits_int32(heads, k_stride_head_bytes, 2 * (int64_t)head_dim) ||
      !span_fits_int32(heads, v_stride_head_bytes, 2 * (int64_t)head_dim) ||
      !span_fits_int32(heads, kc_stride_head_bytes, head_dim) ||
      !span_fits_int32(heads, vc_stride_head_bytes, head_dim))
    return KVSTORE_ERR_SHAPE;
  // Largest byte offset within a cache (last page, last slot of a page, plus
  // the in-slot span of at most INT32_MAX checked above) must fit in int64,
  // whether the slot is addressed as page/offset or linearly.
  const int64_t max_page = (size_limit - 1) / page_size;
  if (!fits(max_page + 1, kc_stride_page_bytes) || !fits(max_page + 1, vc_stride_page_bytes) ||
      !fits(page_size, kc_stride_offset_bytes) || !fits(page_size, vc_stride_offset_bytes) ||
      !fits(size_limit, kc_stride_offset_bytes) || !fits(size_limit, vc_stride_offset_bytes) ||
      !sum_fits(max_page * kc_stride_page_bytes, page_size * kc_stride_offset_bytes, INT32_MAX) ||
      !sum_fits(max_page * vc_stride_page_bytes, page_size * vc_stride_offset_bytes, INT32_MAX) ||
      !sum_fits(size_limit * kc_stride_offset_bytes, INT32_MAX, 0) ||
      !sum_fits(size_limit * vc_stride_offset_bytes, INT32_MAX, 0))
    return KVSTORE_ERR_SHAPE;
  if (!fits(batch, k_stride_token_bytes) || !fits(batch, v_stride_token_bytes))
    return KVSTORE_ERR_SHAPE;
  const int ic = check_index_args(indices, idx_dtype, idx_stride, batch);
  if (ic != KVSTORE_OK) return ic;
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16))
    return KVSTORE_ERR_ALIGN;
  const int64_t units = heads * (head_dim / 16);
  if (units > INT32_MAX) return KVSTORE_ERR_SHAPE;

  p.k = static_cast<const uint8_t*>(k);
  p.v = static_cast<const uint8_t*>(v);
  p.k_cache = static_cast<uint8_t*>(k_cache);
  p.v_cache = static_cast<uint8_t*>(v_cache);
  p.indices = indices;
  p.inv_k = nullptr;
  p.inv_v = nullptr;
  p.idx_stride = idx_stride;
  p.k_stride_token = k_stride_token_bytes;
  p.k_stride_head = k_stride_head_bytes;
  p.v_stride_token = v_stride_token_bytes;
  p.v_stride_head = v_stride_head_bytes;
  p.kc_stride_page = kc_stride_page_bytes;
  p.kc_stride_offset = kc_stride_offset_bytes;
  p.kc_stride_head = kc_stride_head_bytes;
  p.vc_stride_page = vc_stride_page_bytes;
  p.vc_stride_offset = vc_stride_offset_bytes;
  p.vc_stride_head = vc_stride_head_bytes;
  p.size_limit = size_limit;
  p.page_size = page_size;
  p.batch = batch;
  p.units_per_head = (uint32_t)(head_dim / 16);
  p.units = (uint32_t)units;
  p.page_shift = -1;
  if ((page_size & (page_size - 1)) == 0) {
    int sh = 0;
    while ((int64_t(1) << sh) < page_size) ++sh;
    p.page_shift = sh;
  }
  p.linear_pages = (kc_stride_page_bytes == page_size * kc_stride_offset_bytes &&
                    vc_stride_page_bytes == page_size * vc_stride_offset_bytes)
                       ? 1
                       : 0;
  return KVSTORE_OK;
}

// Heads are back to back in the input rows and in the cache slots.
bool fp8_flat(const Fp8Params& p, int32_t head_dim) {
  return p.k_stride_head == 2 * (int64_t)head_dim && p.v_stride_head == 2 * (int64_t)head_dim &&
         p.kc_stride_head == head_dim && p.vc_stride_head == head_dim;
}

// The fused store with given per-tensor inverse scales, into e4m3fn or e5m2
// caches.
int fp8_paged_store(bool e5m2, const void* k, const void* v, void* k_cache, void* v_cache,
                    const void* indices, int idx_dtype, int64_t idx_stride, int src_dtype,
                    int32_t num_heads, int32_t head_dim, int64_t k_stride_token_bytes,
                    int64_t k_stride_head_bytes, int64_t v_stride_token_bytes,
                    int64_t v_stride_head_bytes, int64_t kc_stride_page_bytes,
                    int64_t kc_stride_offset_bytes, int64_t kc_stride_head_bytes,
                    int64_t vc_stride_page_bytes, int64_t vc_stride_offset_bytes,
                    int64_t vc_stride_head_bytes, uint32_t batch, int64_t size_limit,
                    int64_t page_size, const float* inv_k_scale_ptr, const float* inv_v_scale_ptr,
                    hipStream_t stream) {
  if (idx_dtype != KVSTORE_IDX_I32 && idx_dtype != KVSTORE_IDX_I64) return KVSTORE_ERR_DTYPE;
  if (src_dtype != KVSTORE_SRC_BF16 && src_dtype != KVSTORE_SRC_FP16) return KVSTORE_ERR_DTYPE;
  if (batch == 0) return KVSTORE_OK;
  Fp8Params p;
  const int st = fill_fp8_params(
      p, k, v, k_cache, v_cache, indices, idx_dtype, idx_stride, num_heads, head_dim,
      k_stride_token_bytes, k_stride_head_bytes, v_stride_token_bytes, v_stride_head_bytes,
      kc_stride_page_bytes, kc_stride_offset_bytes, kc_stride_head_bytes, vc_stride_page_bytes,
      vc_stride_offset_bytes, vc_stride_head_bytes, batch, size_limit, page_size);
  if (st != KVSTORE_OK) return st;
  if (!aligned(inv_k_scale_ptr, 4) || !aligned(inv_v_scale_ptr, 4)) return KVSTORE_ERR_ALIGN;
  p.inv_k = inv_k_scale_ptr;
  p.inv_v = inv_v_scale_ptr;
  const bool flat = fp8_flat(p, head_dim);
  const bool fp16 = src_dtype == KVSTORE_SRC_FP16;
  const bool i64 = idx_dtype == KVSTORE_IDX_I64;

  // Passes of 1024 elements (128 groups of 8, two per lane): up to 2 per wave,
  // wider rows split over blockIdx.y.
  const int64_t waves_units = ceil_div(p.units, kWave);
  const int passes = waves_units >= 2 ? 2 : 1;
  const int64_t slices = ceil_div(waves_units, passes);
  if (2 * slices > kMaxGridY) return KVSTORE_ERR_SHAPE;
  return launch_in_runs(p, p.token_base, p.batch, batch, [&](const Fp8Params& run) {
    const dim3 grid((uint32_t)ceil_div(run.batch, kWavesPerBlock), (uint32_t)(2 * slices));
    return passes == 2 ? launch_fp8_passes<2>(run, flat, fp16, i64, e5m2, grid, stream)
                       : launch_fp8_passes<1>(run, flat, fp16, i64, e5m2, grid, stream);
  });
}

}  // namespace

extern "C" {

int kvstore_copy(const void* k, const void* v, void* k_cache, void* v_cache,
                 const void* indices, int idx_dtype, int64_t idx_stride, int64_t row_bytes,
                 int64_t k_stride_bytes, int64_t v_stride_bytes, int64_t cache_stride_bytes,
                 uint32_t batch, int64_t size_limit, hipStream_t stream) {
  if (idx_dtype != KVSTORE_IDX_I32 && idx_dtype != KVSTORE_IDX_I64) return KVSTORE_ERR_DTYPE;
  if (batch == 0) return KVSTORE_OK;
  if (!k || !v || !k_cache || !v_cache || !indices) return KVSTORE_ERR_NULL;
  if (row_bytes <= 0 || row_bytes > INT32_MAX || row_bytes % 4) return KVSTORE_ERR_SHAPE;
  if (k_stride_bytes < 0 || v_stride_bytes < 0 || cache_stride_bytes < row_bytes)
    return KVSTORE_ERR_SHAPE;
  if (size_limit <= 0 || !fits(size_limit, cache_stride_bytes)) return KVSTORE_ERR_SHAPE;
  if (!fits(batch, k_stride_bytes) || !fits(batch, v_stride_bytes)) return KVSTORE_ERR_SHAPE;
  const int ic = check_index_args(indices, idx_dtype, idx_stride, batch);
  if (ic != KVSTORE_OK) return ic;
  // Widest lane vector (16, 8 or 4 bytes) that every row start and the row
  // size allow.
  const uintptr_t bits = (uintptr_t)k | (uintptr_t)v | (uintptr_t)k_cache | (uintptr_t)v_cache |
                         (uintptr_t)k_stride_bytes | (uintptr_t)v_stride_bytes |
                         (uintptr_t)cache_stride_bytes | (uintptr_t)row_bytes;
  const int vw = (bits % 16 == 0) ? 16 : (bits % 8 == 0) ? 8 : (bits % 4 == 0) ? 4 : 0;
  if (vw == 0) return KVSTORE_ERR_ALIGN;

  CopyParams p;
  p.k = static_cast<const uint8_t*>(k);
  p.v = static_cast<const uint8_t*>(v);
  p.k_cache = static_cast<uint8_t*>(k_cache);
  p.v_cache = static_cast<uint8_t*>(v_cache);
  p.indices = indices;
  p.idx_stride = idx_stride;
  p.k_stride = k_stride_bytes;
  p.v_stride = v_stride_bytes;
  p.cache_stride = cache_stride_bytes;
  p.size_limit = size_limit;
  p.row_bytes = (uint32_t)row_bytes;
  return launch_in_runs(p, p.token_base, p.batch, batch, [&](const CopyParams& run) {
    return idx_dtype == KVSTORE_IDX_I64 ? launch_copy<int64_t>(run, vw, stream)
                                        : launch_copy<int32_t>(run, vw, stream);
  });
}

int kvstore_fp8_paged(const void* k, const void* v, void* k_cache, void* v_cache,
                      const void* indices, int idx_dtype, int64_t idx_stride, int src_dtype,
                      int32_t num_heads, int32_t head_dim, int64_t k_stride_token_bytes,
                      int64_t k_stride_head_bytes, int64_t v_stride_token_bytes,
                      int64_t v_stride_head_bytes, int64_t kc_stride_page_bytes,
                      int64_t kc_stride_offset_bytes, int64_t kc_stride_head_bytes,
                      int64_t vc_stride_page_bytes, int64_t vc_stride_offset_bytes,
                      int64_t vc_stride_head_bytes, uint32_t batch, int64_t size_limit,
                      int64_t page_size, const float* inv_k_scale_ptr,
                      const float* inv_v_scale_ptr, hipStream_t stream) {
  return fp8_paged_store(false, k, v, k_cache, v_cache, indices, idx_dtype, idx_stride,
                         src_dtype, num_heads, head_dim, k_stride_token_bytes,
                         k_stride_head_bytes, v_stride_token_bytes, v_stride_head_bytes,
                         kc_stride_page_bytes, kc_stride_offset_bytes, kc_stride_head_bytes,
                         vc_stride_page_bytes, vc_stride_offset_bytes, vc_stride_head_bytes,
                         batch, size_limit, page_size, inv_k_scale_ptr, inv_v_scale_ptr, stream);
}

int kvstore_fp8_paged_e5m2(const void* k, const void* v, void* k_cache, void* v_cache,
                           const void* indices, int idx_dtype, int64_t idx_stride, int src_dtype,
                           int32_t num_heads, int32_t head_dim, int64_t k_stride_token_bytes,
                           int64_t k_stride_head_bytes, int64_t v_stride_token_bytes,
                           int64_t v_stride_head_bytes, int64_t kc_stride_page_bytes,
                           int64_t kc_stride_offset_bytes, int64_t kc_stride_head_bytes,
                           int64_t vc_stride_page_bytes, int64_t vc_stride_offset_bytes,
                           int64_t vc_stride_head_bytes, uint32_t batch, int64_t size_limit,
                           int64_t page_size, const float* inv_k_scale_ptr,
                           const float* inv_v_scale_ptr, hipStream_t stream) {
  return fp8_paged_store(true, k, v, k_cache, v_cache, indices, idx_dtype, idx_stride,
                         src_dtype, num_heads, head_dim, k_stride_token_bytes,
                         k_stride_head_bytes, v_stride_token_bytes, v_stride_head_bytes,
                         kc_stride_page_bytes, kc_stride_offset_bytes, kc_stride_head_bytes,
                         vc_stride_page_bytes, vc_stride_offset_bytes, vc_stride_head_bytes,
                         batch, size_limit, page_size, inv_k_scale_ptr, inv_v_scale_ptr, stream);
}

int kvstore_fp8_paged_dynamic(const void* k, const void* v, void* k_cache, void* v_cache,
                              const void* indices, int idx_dtype, int64_t idx_stride,
                              int src_dtype, int32_t num_heads, int32_t head_dim,
                              int64_t k_stride_token_bytes, int64_t k_stride_head_bytes,
                              int64_t v_stride_token_bytes, int64_t v_stride_head_bytes,
                              int64_t kc_stride_page_bytes, int64_t kc_stride_offset_bytes,
                              int64_t kc_stride_head_bytes, int64_t vc_stride_page_bytes,
                              int64_t vc_stride_offset_bytes, int64_t vc_stride_head_bytes,
                              float* k_scale_cache, float* v_scale_cache, int granularity,
                              int64_t ks_stride_page_bytes, int64_t ks_stride_offset_bytes,
                              int64_t ks_stride_head_bytes, int64_t vs_stride_page_bytes,
                              int64_t vs_stride_offset_bytes, int64_t vs_stride_head_bytes,
                              uint32_t batch, int64_t size_limit, int64_t page_size,
                              hipStream_t stream) {
  if (idx_dtype != KVSTORE_IDX_I32 && idx_dtype != KVSTORE_IDX_I64) return KVSTORE_ERR_DTYPE;
  if (src_dtype != KVSTORE_SRC_BF16 && src_dtype != KVSTORE_SRC_FP16) return KVSTORE_ERR_DTYPE;
  if (granularity != KVSTORE_SCALE_PER_TOKEN && granularity != KVSTORE_SCALE_PER_TOKEN_HEAD)
    return KVSTORE_ERR_DTYPE;
  if (batch == 0) return KVSTORE_OK;
  Fp8DynParams d;
  const int st = fill_fp8_params(
      d.base, k, v, k_cache, v_cache, indices, idx_dtype, idx_stride, num_heads, head_dim,
      k_stride_token_bytes, k_stride_head_bytes, v_stride_token_bytes, v_stride_head_bytes,
      kc_stride_page_bytes, kc_stride_offset_bytes, kc_stride_head_bytes, vc_stride_page_bytes,
      vc_stride_offset_bytes, vc_stride_head_bytes, batch, size_limit, page_size);
  if (st != KVSTORE_OK) return st;
  if (!k_scale_cache || !v_scale_cache) return KVSTORE_ERR_NULL;
  const bool per_head = granularity == KVSTORE_SCALE_PER_TOKEN_HEAD;
  // The whole row must sit in one wave: at most kMaxDynPasses * 64 units.
  if (d.base.units > (uint32_t)(kMaxDynPasses * kWave)) return KVSTORE_ERR_SHAPE;
  // Per-head groups are reduced within aligned lane groups.
  const uint32_t uph = d.base.units_per_head;
  if (per_head && (uph > (uint32_t)kWave || (uph & (uph - 1)) != 0)) return KVSTORE_ERR_SHAPE;
  const int64_t sstrides[6] = {ks_stride_page_bytes, ks_stride_offset_bytes,
                               ks_stride_head_bytes, vs_stride_page_bytes,
                               vs_stride_offset_bytes, vs_stride_head_bytes};
  for (int64_t s : sstrides) {
    if (s < 0) return KVSTORE_ERR_SHAPE;
    if (!aligned(s, 4)) return KVSTORE_ERR_ALIGN;
  }
  if (!aligned(k_scale_cache, 4) || !aligned(v_scale_cache, 4)) return KVSTORE_ERR_ALIGN;
  const int64_t groups = per_head ? num_heads : 1;
  const int64_t max_page = (size_limit - 1) / page_size;
  if (!fits(max_page + 1, ks_stride_page_bytes) || !fits(max_page + 1, vs_stride_page_bytes) ||
      !fits(page_size, ks_stride_offset_bytes) || !fits(page_size, vs_stride_offset_bytes) ||
      !fits(groups, ks_stride_head_bytes) || !fits(groups, vs_stride_head_bytes) ||
      !sum_fits(max_page * ks_stride_page_bytes, page_size * ks_stride_offset_bytes,
                groups * ks_stride_head_bytes) ||
      !sum_fits(max_page * vs_stride_page_bytes, page_size * vs_stride_offset_bytes,
                groups * vs_stride_head_bytes))
    return KVSTORE_ERR_SHAPE;

  d.k_scales = reinterpret_cast<uint8_t*>(k_scale_cache);
  d.v_scales = reinterpret_cast<uint8_t*>(v_scale_cache);
  d.ks_stride_page = ks_stride_page_bytes;
  d.ks_stride_offset = ks_stride_offset_bytes;
  d.ks_stride_head = ks_stride_head_bytes;
  d.vs_stride_page = vs_stride_page_bytes;
  d.vs_stride_offset = vs_stride_offset_bytes;
  d.vs_stride_head = vs_stride_head_bytes;
  const bool flat = fp8_flat(d.base, head_dim);
  const bool fp16 = src_dtype == KVSTORE_SRC_FP16;
  const bool i64 = idx_dtype == KVSTORE_IDX_I64;
  const int64_t waves_units = ceil_div(d.base.units, kWave);
  return launch_in_runs(d, d.base.token_base, d.base.batch, batch, [&](const Fp8DynParams& run) {
    const dim3 grid((uint32_t)ceil_div(run.base.batch, kDynWavesPerBlock), 2);
    if (waves_units <= 1) return launch_dyn_passes<1>(run, per_head, flat, fp16, i64, grid, stream);
    if (waves_units <= 2) return launch_dyn_passes<2>(run, per_head, flat, fp16, i64, grid, stream);
    return launch_dyn_passes<4>(run, per_head, flat, fp16, i64, grid, stream);
  });
}

int kvstore_check_error(hipStream_t stream, int64_t* first_bad_token, uint64_t* bad_count) {
  // The flag is taken by the same one-thread kernel as kvstore_take_error, in
  // stream order, into a per-device result word pair that one check at a time
  // uses; then the stream is waited for and the pair read.
  static std::mutex one_check;
  std::lock_guard<std::mutex> hold(one_check);
  int64_t* taken = nullptr;
  if (hipGetSymbolAddress(reinterpret_cast<void**>(&taken), HIP_SYMBOL(g_kvstore_taken)) !=
      hipSuccess)
    return KVSTORE_ERR_HIP;
  if (launch(kvstore_take_error_kernel, dim3(1), dim3(1), 0, stream, taken) != KVSTORE_OK)
    return KVSTORE_ERR_HIP;
  int64_t h[2];
  if (hipMemcpyAsync(h, taken, sizeof h, hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return KVSTORE_ERR_HIP;
  if (first_bad_token) *first_bad_token = h[0];
  if (bad_count) *bad_count = (uint64_t)h[1];
  return h[1] ? KVSTORE_ERR_OOB : KVSTORE_OK;
}

int kvstore_take_error(int64_t* out_device, hipStream_t stream) {
  if (!out_device) return KVSTORE_ERR_NULL;
  if (!aligned(out_device, 8)) return KVSTORE_ERR_ALIGN;
  return launch(kvstore_take_error_kernel, dim3(1), dim3(1), 0, stream, out_device);
}

const char* kvstore_strerror(int status) {
  switch (status) {
    case KVSTORE_OK: return "ok";
    case KVSTORE_ERR_NULL: return "a required pointer is NULL";
    case KVSTORE_ERR_SHAPE: return "a size or stride is out of range";
    case KVSTORE_ERR_ALIGN: return "a pointer or stride is not aligned as required";
    case KVSTORE_ERR_DTYPE: return "unknown index or source type";
    case KVSTORE_ERR_HIP: return "HIP runtime error";
    case KVSTORE_ERR_OOB: return "an index was outside [0, size_limit); its row was skipped";
    default: return "unknown status";
  }
}

}  // extern "C"
