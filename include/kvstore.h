/*
 * libkvstore -- KV-cache store for MI355X (gfx950).
 *
 * Four store operations and their error reporting, as a plain C ABI.  Every
 * pointer argument of a store call is a DEVICE pointer owned by the caller
 * (for example a torch tensor's data pointer); the library never allocates,
 * frees or synchronises inside a store call.  Work is enqueued on the given
 * HIP stream of the current device and returns immediately, so store calls
 * may be captured into a HIP graph.
 *
 * Operations and the passages that define them:
 *
 *   kvstore_copy       -- sglang "kvcache.cuh" (JIT elementwise kernel),
 *                         store_kvcache / copy_kv_warp and the host run():
 *                         for each token t, the K row and the V row of t are
 *                         copied byte for byte into row indices[t] of the K
 *                         and V caches; the index must lie in [0, size_limit).
 *   kvstore_fp8_paged  -- sglang "trtllm_fp8_kv_kernel.py",
 *                         _fused_fp8_set_kv_buffer_kernel, _process_kv_tensor
 *                         and the wrapper fused_fp8_set_kv_buffer: for token t
 *                         with loc = indices[t], page = loc / page_size and
 *                         offset = loc % page_size; every element x of K (V)
 *                         becomes e4m3fn(x * inv_k) (e4m3fn(x * inv_v)) at
 *                         [page, offset, head, dim] of the K (V) cache.
 *   kvstore_fp8_paged_e5m2 -- the same store into float8_e5m2 caches, which
 *                         the page's unfused path also writes.
 *   kvstore_fp8_paged_dynamic -- the same store with per-token (or per token
 *                         and head) scales computed in the kernel: the module
 *                         docstring of "trtllm_fp8_kv_kernel.py" counts scale
 *                         computation (per token, and per page) among the
 *                         fused kernel's steps.
 *
 * Numerics of kvstore_fp8_paged: x (bf16 or fp16) is widened to fp32 exactly,
 * multiplied once in fp32 (round to nearest) by the inverse scale, and
 * rounded to the nearest e4m3fn value with ties to even; values beyond +-448
 * (including infinities) saturate to +-448, NaN stays NaN (0x7F | sign).
 * The page leaves rounding and overflow of its float8 cast unstated; this is
 * the reading the library implements, bit-exactly.
 *
 * Out-of-range indices: the page's copy kernel asserts on them and its fused
 * kernel does not check them at all.  Here a token whose index is outside
 * [0, size_limit) is skipped (neither its K nor its V row is written, every
 * other token is) and recorded in a per-device error flag, read and cleared
 * by kvstore_check_error (which synchronises) or, in stream order and inside
 * a captured graph, by kvstore_take_error.  Store calls report only argument
 * errors.
 *
 * Indices must be unique within one call: two tokens naming the same slot
 * race, and which one lands is undefined (as on the pages).
 *
 * Concurrency: the error flag is one per device and is shared by every store
 * call on that device; calls may run concurrently on several streams.  Each
 * rejected token is recorded by one atomic update of the flag and each check
 * or take clears it by one atomic exchange, so a report made while a check or
 * take runs on another stream lands, whole, in that one or in the next.  The
 * count of rejected tokens saturates at 2^32 - 1 between two checks.
 */
#ifndef KVSTORE_H
#define KVSTORE_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Index element types. */
enum { KVSTORE_IDX_I32 = 0, KVSTORE_IDX_I64 = 1 };

/* Source element types of kvstore_fp8_paged / kvstore_fp8_paged_dynamic. */
enum { KVSTORE_SRC_BF16 = 0, KVSTORE_SRC_FP16 = 1 };

/* Scale groups of kvstore_fp8_paged_dynamic. */
enum { KVSTORE_SCALE_PER_TOKEN = 0, KVSTORE_SCALE_PER_TOKEN_HEAD = 1 };

/* Status codes.  Negative codes returned by a store call mean nothing was
 * launched and no memory was touched, with one exception: a batch above 2^24
 * tokens runs as several launches (see `batch` below), and KVSTORE_ERR_HIP
 * from a later launch leaves the earlier runs queued. */
enum {
  KVSTORE_OK = 0,
  KVSTORE_ERR_NULL = -1,  /* a required pointer is NULL */
  KVSTORE_ERR_SHAPE = -2, /* a size or stride is out of range */
  KVSTORE_ERR_ALIGN = -3, /* a pointer or stride breaks the alignment rule */
  KVSTORE_ERR_DTYPE = -4, /* unknown index or source type code */
  KVSTORE_ERR_HIP = -5,   /* the HIP runtime reported an error */
  KVSTORE_ERR_OOB = -6    /* (kvstore_check_error) some index was out of range */
};

/*
 * Scatter copy (sglang "kvcache.cuh", store_kvcache).
 *
 *   k, v         device, [batch] rows of row_bytes bytes, row t at
 *                k + t * k_stride_bytes (v likewise).  Read only.
 *   k_cache,     device, rows of row_bytes bytes at
 *   v_cache      cache + slot * cache_stride_bytes (one stride for both, as
 *                on the page).  Written only at the slots named by indices.
 *   indices      device, element t at indices[t * idx_stride], of type
 *                idx_dtype (KVSTORE_IDX_I32 / KVSTORE_IDX_I64).
 *   idx_stride   in elements, >= 1.
 *   row_bytes    bytes per K (and V) row: > 0, a multiple of 4, < 2^31, and
 *                at most 65535 * 4 * 64 lane vectors (268,431,360 bytes with
 *                16-byte lanes, 134,215,680 with 8-byte, 67,107,840 with
 *                4-byte lanes; longer rows return KVSTORE_ERR_SHAPE).
 *   *_stride_bytes  multiples of 4; k/v strides >= 0,
 *                cache_stride_bytes >= row_bytes.
 *   batch        number of tokens; 0 returns KVSTORE_OK and launches nothing.
 *                Above 2^24 tokens the call queues one launch per run of at
 *                most 2^24 tokens, in token order, on `stream` (the grid of
 *                one launch stays far below 2^32 work-items); token positions
 *                in the flag stay those of the whole batch.
 *   size_limit   valid slots are [0, size_limit); > 0, and
 *                size_limit * cache_stride_bytes must fit in int64.
 *   stream       HIP stream of the current device (0 = null stream).
 *
 * Alignment: k, v, k_cache, v_cache 4-byte aligned; indices aligned to its
 * element size.  Lanes move 16 bytes when the row size, the four pointers and
 * the three strides are all multiples of 16 (the fast path), else 8 or 4
 * bytes, as the page's kernel picks its vector width from the row size.  Rows
 * of at most 32 lane vectors are packed several to a 64-lane wave.
 * Element data is never interpreted, so any element type works.
 * Returns KVSTORE_OK or a negative status (nothing launched).
 */
int kvstore_copy(const void* k, const void* v, void* k_cache, void* v_cache,
                 const void* indices, int idx_dtype, int64_t idx_stride,
                 int64_t row_bytes, int64_t k_stride_bytes, int64_t v_stride_bytes,
                 int64_t cache_stride_bytes, uint32_t batch, int64_t size_limit,
                 hipStream_t stream);

/*
 * Fused FP8 (e4m3fn) quantise + paged store (sglang "trtllm_fp8_kv_kernel.py",
 * _fused_fp8_set_kv_buffer_kernel).
 *
 *   k, v         device, [batch, num_heads, head_dim] elements of src_dtype
 *                (KVSTORE_SRC_BF16 / KVSTORE_SRC_FP16); element (t, h, d) at
 *                byte offset t * *_stride_token_bytes + h * *_stride_head_bytes
 *                + 2 * d (dim stride is one element).  Read only.
 *   k_cache,     device, e4m3fn bytes; element (page, off, h, d) at byte offset
 *   v_cache      page * *c_stride_page_bytes + off * *c_stride_offset_bytes
 *                + h * *c_stride_head_bytes + d.  Both the page's 4-D
 *                [pages, page_size, H, D] cache and its flat [slots, H, D]
 *                cache (page stride = page_size * slot stride) are expressed
 *                this way.
 *   indices, idx_dtype, idx_stride, batch, size_limit, stream: as in
 *                kvstore_copy; size_limit is normally num_pages * page_size.
 *   num_heads    > 0;  head_dim > 0 and a multiple of 16;  num_heads *
 *                head_dim <= 67,106,816 elements, and the byte offset of the
 *                last head's end within a token row or a slot below 2^31
 *                (else KVSTORE_ERR_SHAPE).
 *   page_size    > 0 (any value; powers of two take a shift).
 *   inv_k_scale_ptr, inv_v_scale_ptr
 *                device pointers to one fp32 inverse scale each, or NULL for
 *                1.0 (no scaling).  Each is independent.  Read on the device,
 *                so the call never waits on the host.
 *
 * Alignment: k, v and their token/head strides 16-byte aligned; k_cache,
 * v_cache and their page/offset/head strides 16-byte aligned; indices aligned
 * to its element size; scale pointers 4-byte aligned.  Strides >= 0; the cache
 * layout must not overlap itself (offset stride >= heads * head stride when
 * heads are inside a slot is NOT checked: overlapping layouts race).
 * Returns KVSTORE_OK or a negative status (nothing launched).
 */
int kvstore_fp8_paged(const void* k, const void* v, void* k_cache, void* v_cache,
                      const void* indices, int idx_dtype, int64_t idx_stride, int src_dtype,
                      int32_t num_heads, int32_t head_dim, int64_t k_stride_token_bytes,
                      int64_t k_stride_head_bytes, int64_t v_stride_token_bytes,
                      int64_t v_stride_head_bytes, int64_t kc_stride_page_bytes,
                      int64_t kc_stride_offset_bytes, int64_t kc_stride_head_bytes,
                      int64_t vc_stride_page_bytes, int64_t vc_stride_offset_bytes,
                      int64_t vc_stride_head_bytes, uint32_t batch, int64_t size_limit,
                      int64_t page_size, const float* inv_k_scale_ptr,
                      const float* inv_v_scale_ptr, hipStream_t stream);

/*
 * As kvstore_fp8_paged, into float8_e5m2 caches (the page's unfused path,
 * _naive_fp8_set_kv_buffer in "trtllm_fp8_kv_kernel.py", stores into e5m2 as
 * well as e4m3fn caches).  Same arguments and rules; each element becomes the
 * nearest e5m2 value to x * inv (1 sign, 5 exponent bits with bias 15, 2
 * mantissa bits), ties to even, saturating to +-57344 (infinities too), NaN
 * -> 0x7F | sign.
 */
int kvstore_fp8_paged_e5m2(const void* k, const void* v, void* k_cache, void* v_cache,
                           const void* indices, int idx_dtype, int64_t idx_stride, int src_dtype,
                           int32_t num_heads, int32_t head_dim, int64_t k_stride_token_bytes,
                           int64_t k_stride_head_bytes, int64_t v_stride_token_bytes,
                           int64_t v_stride_head_bytes, int64_t kc_stride_page_bytes,
                           int64_t kc_stride_offset_bytes, int64_t kc_stride_head_bytes,
                           int64_t vc_stride_page_bytes, int64_t vc_stride_offset_bytes,
                           int64_t vc_stride_head_bytes, uint32_t batch, int64_t size_limit,
                           int64_t page_size, const float* inv_k_scale_ptr,
                           const float* inv_v_scale_ptr, hipStream_t stream);

/*
 * Fused FP8 (e4m3fn) quantise + paged store with dynamic scales.  The
 * docstring of sglang "trtllm_fp8_kv_kernel.py" lists per-token scale
 * computation among the fused kernel's steps (its code only applies a given
 * per-tensor scale); this call computes the scales itself.
 *
 * For each valid token and each of K and V, the scale groups are the whole
 * row (granularity KVSTORE_SCALE_PER_TOKEN) or each head
 * (KVSTORE_SCALE_PER_TOKEN_HEAD).  Per group: amax = max |x| (NaN elements
 * ignored); scale = max(amax / 448, 2^-126) in fp32 (correctly rounded; the
 * floor keeps 1/scale finite); inv = 1 / scale in fp32; every element becomes
 * e4m3fn(x * inv) with the rules of kvstore_fp8_paged; and the fp32 scale of
 * group g is written at byte offset page * *s_stride_page_bytes +
 * off * *s_stride_offset_bytes + g * *s_stride_head_bytes of k_scale_cache /
 * v_scale_cache (the head stride is unused per token).  Dequantisation is
 * code value * scale.
 *
 *   All other arguments: as in kvstore_fp8_paged.
 *   k_scale_cache, v_scale_cache  device fp32 arrays, 4-byte aligned; scale
 *                strides >= 0 and multiples of 4.
 * Limits: num_heads * head_dim <= 4096 (one 64-lane wave holds the whole
 * row); per head additionally head_dim in {16, 32, 64, ..., 1024}.  Larger
 * shapes return KVSTORE_ERR_SHAPE.  Unknown granularity: KVSTORE_ERR_DTYPE.
 */
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
                              hipStream_t stream);

/*
 * Waits for `stream`, then reads and clears the current device's error flag.
 * Returns KVSTORE_OK when no store since the last check saw an out-of-range
 * index, KVSTORE_ERR_OOB when some did, KVSTORE_ERR_HIP on a runtime error.
 * first_bad_token (nullable) receives the smallest rejected token position of
 * any call since the last check, or -1; bad_count (nullable) the number of
 * rejected tokens.  This is the only call that synchronises: it enqueues the
 * flag's take on `stream` (after the stream's earlier work), then waits for
 * the stream.  The flag is per device and shared by all streams: reports of
 * stores still running on other streams are counted by this check or by the
 * next, never split or lost.  Calls from several host threads are serialised.
 */
int kvstore_check_error(hipStream_t stream, int64_t* first_bad_token, uint64_t* bad_count);

/*
 * Graph-capturable form of kvstore_check_error: enqueues on `stream` a
 * one-thread kernel that takes the current device's error flag into
 * `out_device` and clears it, without waiting.  out_device points to two
 * int64 in device memory (8-byte aligned): out_device[0] receives the smallest
 * rejected token position since the last take or check, or -1; out_device[1]
 * the number of rejected tokens.  Stores issued earlier on the same stream are
 * included; the caller reads the two values whenever it synchronises (for
 * example after replaying a graph that captured stores and this call).  The
 * flag is shared by all streams of the device, as for kvstore_check_error.
 * Returns KVSTORE_OK, KVSTORE_ERR_NULL, KVSTORE_ERR_ALIGN or KVSTORE_ERR_HIP
 * (nothing launched).
 */
int kvstore_take_error(int64_t* out_device, hipStream_t stream);

/* Static, human-readable text for a status code. */
const char* kvstore_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* KVSTORE_H */
