// Plain reference kernels for bench.py: same-GPU ceilings for the memory
// shapes of the two store kernels, with nothing of the store in them (no
// index, no scatter, no conversion), each in the fastest form measured on
// gfx950 with non-constant data.  Measurement infrastructure only; the store
// library does not use them.
//
//   bench_plain_copy         contiguous copy of `bytes` bytes: one 64-lane
//                            wave per 2 KiB (two 1 KiB wave accesses),
//                            blocks of 2 waves, non-temporal 16-byte loads
//                            and stores, full occupancy.
//   bench_plain_copy_chunks  the same copy with `chunks` (2, 4 or 8) 1 KiB
//                            wave accesses per wave: small copies run
//                            faster with more bytes per wave (fewer waves
//                            to dispatch), large ones with 2; all of a
//                            wave's loads are issued before its first wait.
//   bench_plain_read2_write1 `waves` waves, each reading 2 KiB of src and
//                            writing 1 KiB to dst (the two halves XORed),
//                            contiguous: the FP8 store's per-wave shape
//                            (2 KiB of bf16 in, 1 KiB of e4m3fn out), written
//                            as it writes (8-byte sc1 buffer stores, lane l
//                            storing bytes [8l, 8l + 8) and [512 + 8l,
//                            520 + 8l) of the wave's 1 KiB).
//   bench_plain_read         reads `bytes` bytes of src, one wave per 2 KiB,
//                            non-temporal; a wave writes one 16-byte word to
//                            sink only if its XOR of the data equals `magic`
//                            (so the loads cannot be dropped, and the
//                            kernel's traffic is its reads alone).
//   bench_plain_write        writes `bytes` bytes of dst, one wave per 4 KiB,
//                            16-byte sc1 buffer stores (measured faster than
//                            non-temporal ones for streaming writes); 16-byte
//                            word i holds a hash of i and `value`.
//   bench_plain_scatter_write one hashed row of `row_bytes` (a multiple of
//                            16, at most 4 KiB) to slot idx[t] of k_cache
//                            and of v_cache for each of `tokens` int32
//                            indices (bench_plain_scatter_write_i64: int64
//                            indices): a store's destinations with no reads
//                            at all (one
//                            wave per row, blocks of 2 waves, K and V over
//                            grid z, 16-byte sc1 buffer stores: the fastest
//                            of sc1, non-temporal and default stores with 1,
//                            2 or 4 rows per wave; at most `waves_per_cu`
//                            waves resident
//                            per CU when non-zero, by a dynamic LDS
//                            allocation the kernel never touches).  Rows
//                            whose index lies outside [0, slots) are skipped.
//
// The data written matters on this GPU: writing all-zero lines measured
// faster than writing varied data, so the callers fill sources with random
// bytes and the write-only kernel writes a hash.
//
// All return 0 when launched, -1 for bad arguments (nothing launched), -5
// when the launch failed.  src, dst and sink are device pointers, 16-byte
// aligned (sink: 64 words of 16 bytes).
#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Raw buffer descriptor over [base, base + 2^31): stride 0, CDNA data format word.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, 0x7FFFFFFF, 0x00020000);
}

// sc1 cache policy: bit 4 of the buffer cache-policy operand.
constexpr int kSc1 = 16;

__global__ __launch_bounds__(128) void plain_copy(const u32x4* __restrict__ s,
                                                  u32x4* __restrict__ d, uint64_t n16) {
  const uint64_t base = ((uint64_t)blockIdx.x * 2 + threadIdx.x / kWave) * (2 * kWave) +
                        threadIdx.x % kWave;
  u32x4 r[2];
#pragma unroll
  for (int c = 0; c < 2; ++c)
    if (base + c * kWave < n16) r[c] = __builtin_nontemporal_load(s + base + c * kWave);
#pragma unroll
  for (int c = 0; c < 2; ++c)
    if (base + c * kWave < n16) __builtin_nontemporal_store(r[c], d + base + c * kWave);
}

__global__ __launch_bounds__(128) void plain_read2_write1(const u32x4* __restrict__ s,
                                                          uint8_t* __restrict__ d, uint64_t waves) {
  const uint64_t w = (uint64_t)blockIdx.x * 2 + threadIdx.x / kWave;
  const uint32_t lane = threadIdx.x % kWave;
  if (w >= waves) return;
  const u32x4* src = s + w * 128;              // 2 KiB = 128 x 16 B
  const u32x4 x = __builtin_nontemporal_load(src + lane) ^
                  __builtin_nontemporal_load(src + kWave + lane);
  const __amdgpu_buffer_rsrc_t r = rsrc(d + w * 1024);
  __builtin_amdgcn_raw_buffer_store_b64(u32x2{x.x, x.y}, r, (int)(lane * 8u), 0, kSc1);
  __builtin_amdgcn_raw_buffer_store_b64(u32x2{x.z, x.w}, r, (int)(512u + lane * 8u), 0, kSc1);
}

__global__ __launch_bounds__(128) void plain_read(const u32x4* __restrict__ s,
                                                  u32x4* __restrict__ sink, uint64_t n16,
                                                  uint32_t magic) {
  const uint64_t base = ((uint64_t)blockIdx.x * 2 + threadIdx.x / kWave) * (2 * kWave) +
                        threadIdx.x % kWave;
  u32x4 x = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
  for (int c = 0; c < 2; ++c)
    if (base + c * kWave < n16) x ^= __builtin_nontemporal_load(s + base + c * kWave);
  if (x.x == magic && x.y == ~magic) sink[threadIdx.x % kWave] = x;
}

__global__ __launch_bounds__(256) void plain_write(uint8_t* __restrict__ d, uint64_t n16,
                                                   uint32_t value) {
  const uint64_t base = ((uint64_t)blockIdx.x * 4 + threadIdx.x / kWave) * (4 * kWave);
  const uint32_t lane = threadIdx.x % kWave;
  if (base >= n16) return;
  const __amdgpu_buffer_rsrc_t r = rsrc(d + base * 16);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint64_t i = base + c * kWave + lane;
    if (i < n16) {
      const uint32_t h = (uint32_t)i * 0x9E3779B1u ^ value;
      __builtin_amdgcn_raw_buffer_store_b128(u32x4{h, h ^ 0x85EBCA6Bu, h ^ 0xC2B2AE35u,
                                                   h + 0x27D4EB2Fu},
                                             r, (int)((i - base) * 16), 0, kSc1);
    }
  }
}

// kChunks 1 KiB wave accesses per wave; lanes past the end load the last
// 16-byte word (and store nothing), so no load sits under a branch, and an
// empty asm operand per loaded value keeps every load ahead of the first wait.
template <int kChunks>
__global__ __launch_bounds__(128) void plain_copy_n(const u32x4* __restrict__ s,
                                                    u32x4* __restrict__ d, uint64_t n16) {
  const uint64_t base = ((uint64_t)blockIdx.x * 2 + threadIdx.x / kWave) * (kChunks * kWave) +
                        threadIdx.x % kWave;
  u32x4 r[kChunks];
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const uint64_t i = base + c * kWave;
    r[c] = __builtin_nontemporal_load(s + (i < n16 ? i : n16 - 1));
  }
#pragma unroll
  for (int c = 0; c < kChunks; ++c) asm volatile("" : "+v"(r[c]));
#pragma unroll
  for (int c = 0; c < kChunks; ++c)
    if (base + c * kWave < n16) __builtin_nontemporal_store(r[c], d + base + c * kWave);
}

template <typename IdxT>
__global__ __launch_bounds__(128) void plain_scatter_write(uint8_t* __restrict__ kc,
                                                           uint8_t* __restrict__ vc,
                                                           const IdxT* __restrict__ idx,
                                                           uint32_t tokens, uint32_t row16,
                                                           uint64_t cache_stride, int64_t slots,
                                                           uint32_t seed) {
  const uint32_t t = __builtin_amdgcn_readfirstlane(blockIdx.x * 2 + threadIdx.x / kWave);
  if (t >= tokens) return;
  const uint32_t lane = threadIdx.x % kWave;
  const int64_t loc = (int64_t)idx[t];
  if (loc < 0 || loc >= slots) return;
  const __amdgpu_buffer_rsrc_t row = rsrc((blockIdx.z ? vc : kc) + (uint64_t)loc * cache_stride);
  const uint32_t salt = seed ^ (blockIdx.z ? 0x5BD1E995u : 0u);
#pragma unroll
  for (uint32_t c = 0; c < 4; ++c) {
    const uint32_t w = c * kWave + lane;  // 16-byte word of the row
    if (w < row16) {
      const uint32_t h = (t * 0x9E3779B1u + w) ^ salt;
      __builtin_amdgcn_raw_buffer_store_b128(
          u32x4{h, h ^ 0x85EBCA6Bu, h ^ 0xC2B2AE35u, h + 0x27D4EB2Fu}, row, (int)(w * 16), 0,
          kSc1);
    }
  }
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Blocks of `per_block` 16-byte words covering n16; 0 if too many.
uint64_t blocks_for(uint64_t n16, uint64_t per_block) {
  const uint64_t blocks = (n16 + per_block - 1) / per_block;
  return blocks > 0x7FFFFFFFull ? 0 : blocks;
}

}  // namespace

extern "C" int bench_plain_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream) {
  if (!src || !dst || bytes <= 0 || bytes % 16 != 0 || !aligned16(src) || !aligned16(dst))
    return -1;
  const uint64_t n16 = (uint64_t)bytes / 16;
  const uint64_t blocks = blocks_for(n16, 4ull * kWave);
  if (blocks == 0) return -1;
  hipLaunchKernelGGL(plain_copy, dim3((uint32_t)blocks), dim3(128), 0, stream,
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n16);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" int bench_plain_copy_chunks(const void* src, void* dst, int64_t bytes, int chunks,
                                       hipStream_t stream) {
  if (!src || !dst || bytes <= 0 || bytes % 16 != 0 || !aligned16(src) || !aligned16(dst) ||
      (chunks != 2 && chunks != 4 && chunks != 8))
    return -1;
  const uint64_t n16 = (uint64_t)bytes / 16;
  const uint64_t blocks = blocks_for(n16, 2ull * chunks * kWave);
  if (blocks == 0) return -1;
  const u32x4* s = static_cast<const u32x4*>(src);
  u32x4* d = static_cast<u32x4*>(dst);
  if (chunks == 2)
    hipLaunchKernelGGL(plain_copy_n<2>, dim3((uint32_t)blocks), dim3(128), 0, stream, s, d, n16);
  else if (chunks == 4)
    hipLaunchKernelGGL(plain_copy_n<4>, dim3((uint32_t)blocks), dim3(128), 0, stream, s, d, n16);
  else
    hipLaunchKernelGGL(plain_copy_n<8>, dim3((uint32_t)blocks), dim3(128), 0, stream, s, d, n16);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" int bench_plain_read2_write1(const void* src, void* dst, int64_t waves,
                                        hipStream_t stream) {
  if (!src || !dst || waves <= 0 || waves > 0x7FFFFFFFll || !aligned16(src) || !aligned16(dst))
    return -1;
  const uint64_t blocks = ((uint64_t)waves + 1) / 2;
  hipLaunchKernelGGL(plain_read2_write1, dim3((uint32_t)blocks), dim3(128), 0, stream,
                     static_cast<const u32x4*>(src), static_cast<uint8_t*>(dst), (uint64_t)waves);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" int bench_plain_read(const void* src, void* sink, int64_t bytes, uint32_t magic,
                                hipStream_t stream) {
  if (!src || !sink || bytes <= 0 || bytes % 16 != 0 || !aligned16(src) || !aligned16(sink))
    return -1;
  const uint64_t n16 = (uint64_t)bytes / 16;
  const uint64_t blocks = blocks_for(n16, 4ull * kWave);
  if (blocks == 0) return -1;
  hipLaunchKernelGGL(plain_read, dim3((uint32_t)blocks), dim3(128), 0, stream,
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(sink), n16, magic);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" int bench_plain_write(void* dst, int64_t bytes, uint32_t value, hipStream_t stream) {
  if (!dst || bytes <= 0 || bytes % 16 != 0 || !aligned16(dst)) return -1;
  const uint64_t n16 = (uint64_t)bytes / 16;
  const uint64_t blocks = blocks_for(n16, 16ull * kWave);
  if (blocks == 0) return -1;
  hipLaunchKernelGGL(plain_write, dim3((uint32_t)blocks), dim3(256), 0, stream,
                     static_cast<uint8_t*>(dst), n16, value);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

template <typename IdxT>
static int scatter_write(void* k_cache, void* v_cache, const void* idx, int64_t tokens,
                  int64_t row_bytes, int64_t cache_stride, int64_t slots, uint32_t seed,
                  int waves_per_cu, hipStream_t stream) {
  if (!k_cache || !v_cache || !idx || tokens <= 0 || tokens > 0x7FFFFFFFll || row_bytes < 16 ||
      row_bytes > 4096 || row_bytes % 16 != 0 || cache_stride < row_bytes ||
      cache_stride % 16 != 0 || slots <= 0 || !aligned16(k_cache) || !aligned16(v_cache) ||
      ((uintptr_t)idx % sizeof(IdxT)) != 0 || waves_per_cu < 0 || waves_per_cu == 1 ||
      waves_per_cu > 64 || waves_per_cu % 2 != 0)
    return -1;
  uint32_t lds = 0;
  if (waves_per_cu > 0) {
    int dev = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
            hipSuccess ||
        per_cu <= 0)
      return -5;
    // gfx950 allocates LDS to a block in units of 1280 bytes
    lds = (uint32_t)(per_cu / (waves_per_cu / 2) / 1280 * 1280);
  }
  const uint32_t blocks = (uint32_t)((tokens + 1) / 2);
  hipLaunchKernelGGL(plain_scatter_write<IdxT>, dim3(blocks, 1, 2), dim3(128), lds, stream,
                     static_cast<uint8_t*>(k_cache), static_cast<uint8_t*>(v_cache),
                     static_cast<const IdxT*>(idx), (uint32_t)tokens, (uint32_t)(row_bytes / 16),
                     (uint64_t)cache_stride, slots, seed);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" int bench_plain_scatter_write(void* k_cache, void* v_cache, const void* idx,
                                         int64_t tokens, int64_t row_bytes, int64_t cache_stride,
                                         int64_t slots, uint32_t seed, int waves_per_cu,
                                         hipStream_t stream) {
  return scatter_write<int32_t>(k_cache, v_cache, idx, tokens, row_bytes, cache_stride, slots,
                                seed, waves_per_cu, stream);
}

extern "C" int bench_plain_scatter_write_i64(void* k_cache, void* v_cache, const void* idx,
                                             int64_t tokens, int64_t row_bytes,
                                             int64_t cache_stride, int64_t slots, uint32_t seed,
                                             int waves_per_cu, hipStream_t stream) {
  return scatter_write<int64_t>(k_cache, v_cache, idx, tokens, row_bytes, cache_stride, slots,
                                seed, waves_per_cu, stream);
}
