// Plain reference kernels for bench.py: same-GPU ceilings for the memory
// shapes of the two store kernels, with nothing of the store in them (no
// index, no scatter, no conversion).  Measurement infrastructure only; the
// store library does not use them.
//
//   bench_plain_copy         contiguous copy of `bytes` bytes: one 64-lane
//                            wave per 4 KiB (four 1 KiB wave accesses),
//                            non-temporal 16-byte loads and stores, full
//                            occupancy.
//   bench_plain_read2_write1 `waves` waves, each reading 2 KiB of src and
//                            writing 1 KiB to dst (the two halves XORed),
//                            contiguous, non-temporal: the FP8 store's
//                            per-wave shape (2 KiB of bf16 in, 1 KiB of
//                            e4m3fn out).
//   bench_plain_read         reads `bytes` bytes of src, one wave per 4 KiB,
//                            non-temporal; a wave writes one 16-byte word to
//                            sink only if its XOR of the data equals `magic`
//                            (so the loads cannot be dropped, and the
//                            kernel's traffic is its reads alone).
//   bench_plain_write        writes `bytes` bytes of dst, one wave per 4 KiB,
//                            non-temporal; each 16-byte word holds its own
//                            index XOR `value`.
//
// All return 0 when launched, -1 for bad arguments (nothing launched), -5
// when the launch failed.  src, dst and sink are device pointers, 16-byte
// aligned (sink: 64 words of 16 bytes).
#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kChunks = 4;                     // 4 x 1 KiB per copy wave

__global__ __launch_bounds__(256) void plain_copy(const u32x4* __restrict__ s,
                                                  u32x4* __restrict__ d, uint64_t n16) {
  const uint64_t base =
      ((uint64_t)blockIdx.x * 4 + threadIdx.x / kWave) * (kWave * kChunks) + threadIdx.x % kWave;
  u32x4 r[kChunks];
#pragma unroll
  for (int c = 0; c < kChunks; ++c)
    if (base + c * kWave < n16) r[c] = __builtin_nontemporal_load(s + base + c * kWave);
#pragma unroll
  for (int c = 0; c < kChunks; ++c)
    if (base + c * kWave < n16) __builtin_nontemporal_store(r[c], d + base + c * kWave);
}

__global__ __launch_bounds__(128) void plain_read2_write1(const u32x4* __restrict__ s,
                                                          u32x4* __restrict__ d, uint64_t waves) {
  const uint64_t w = (uint64_t)blockIdx.x * 2 + threadIdx.x / kWave;
  const uint32_t lane = threadIdx.x % kWave;
  if (w >= waves) return;
  const u32x4* src = s + w * 128;              // 2 KiB = 128 x 16 B
  const u32x4 a = __builtin_nontemporal_load(src + lane);
  const u32x4 b = __builtin_nontemporal_load(src + kWave + lane);
  __builtin_nontemporal_store(a ^ b, d + w * 64 + lane);   // 1 KiB = 64 x 16 B
}

__global__ __launch_bounds__(256) void plain_read(const u32x4* __restrict__ s,
                                                  u32x4* __restrict__ sink, uint64_t n16,
                                                  uint32_t magic) {
  const uint64_t base =
      ((uint64_t)blockIdx.x * 4 + threadIdx.x / kWave) * (kWave * kChunks) + threadIdx.x % kWave;
  u32x4 r[kChunks];
#pragma unroll
  for (int c = 0; c < kChunks; ++c)
    r[c] = base + c * kWave < n16 ? __builtin_nontemporal_load(s + base + c * kWave)
                                  : u32x4{0u, 0u, 0u, 0u};
  const u32x4 x = r[0] ^ r[1] ^ r[2] ^ r[3];
  if (x.x == magic && x.y == ~magic) sink[threadIdx.x % kWave] = x;
}

__global__ __launch_bounds__(256) void plain_write(u32x4* __restrict__ d, uint64_t n16,
                                                   uint32_t value) {
  const uint64_t base =
      ((uint64_t)blockIdx.x * 4 + threadIdx.x / kWave) * (kWave * kChunks) + threadIdx.x % kWave;
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const uint64_t i = base + c * kWave;
    if (i < n16) {
      const uint32_t w = (uint32_t)i ^ value;
      __builtin_nontemporal_store(u32x4{w, w, w, w}, d + i);
    }
  }
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Blocks of four 4 KiB waves covering n16 16-byte words; 0 if too many.
uint64_t stream_blocks(uint64_t n16) {
  const uint64_t per_block = 4ull * kWave * kChunks;
  const uint64_t blocks = (n16 + per_block - 1) / per_block;
  return blocks > 0x7FFFFFFFull ? 0 : blocks;
}

}  // namespace

extern "C" int bench_plain_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream) {
  if (!src || !dst || bytes <= 0 || bytes % 16 != 0 || !aligned16(src) || !aligned16(dst))
    return -1;
  const uint64_t n16 = (uint64_t)bytes / 16;
  const uint64_t per_block = 4ull * kWave * kChunks;
  const uint64_t blocks = (n16 + per_block - 1) / per_block;
  if (blocks > 0x7FFFFFFFull) return -1;
  hipLaunchKernelGGL(plain_copy, dim3((uint32_t)blocks), dim3(256), 0, stream,
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n16);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" int bench_plain_read2_write1(const void* src, void* dst, int64_t waves,
                                        hipStream_t stream) {
  if (!src || !dst || waves <= 0 || waves > 0x7FFFFFFFll || !aligned16(src) || !aligned16(dst))
    return -1;
  const uint64_t blocks = ((uint64_t)waves + 1) / 2;
  hipLaunchKernelGGL(plain_read2_write1, dim3((uint32_t)blocks), dim3(128), 0, stream,
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), (uint64_t)waves);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" int bench_plain_read(const void* src, void* sink, int64_t bytes, uint32_t magic,
                                hipStream_t stream) {
  if (!src || !sink || bytes <= 0 || bytes % 16 != 0 || !aligned16(src) || !aligned16(sink))
    return -1;
  const uint64_t n16 = (uint64_t)bytes / 16;
  const uint64_t blocks = stream_blocks(n16);
  if (blocks == 0) return -1;
  hipLaunchKernelGGL(plain_read, dim3((uint32_t)blocks), dim3(256), 0, stream,
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(sink), n16, magic);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" int bench_plain_write(void* dst, int64_t bytes, uint32_t value, hipStream_t stream) {
  if (!dst || bytes <= 0 || bytes % 16 != 0 || !aligned16(dst)) return -1;
  const uint64_t n16 = (uint64_t)bytes / 16;
  const uint64_t blocks = stream_blocks(n16);
  if (blocks == 0) return -1;
  hipLaunchKernelGGL(plain_write, dim3((uint32_t)blocks), dim3(256), 0, stream,
                     static_cast<u32x4*>(dst), n16, value);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}
