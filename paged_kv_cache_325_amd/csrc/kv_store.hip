// Slot scatter of fresh K/V rows into the paged cache (gfx950).
//
// The store kernel named in the nano-vllm source study (section 2, attention
// layer) writes each token's k and v rows into the cache at its slot; the
// architecture page ("Prefill- und Decode-Vorbereitung") builds the slots as
// block id * block size + row.  Here a slot of -1 stores nothing.
//
// One thread moves one 16-byte chunk of one (token, kv head) row of K and the
// same chunk of V.  A row is head_dim * elem bytes (256 B for bf16), so 16
// (bf16) or 32 (fp32) consecutive lanes move one row with one dwordx4 load and
// one dwordx4 store each: reads are contiguous per row of the source and each
// destination row is one contiguous 256/512-byte run of the cache.  The copy
// goes through integer registers, so every bit pattern (NaN payloads
// included) is preserved.  HBM-bound: 2 x (read + write) x row bytes per row.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

template <int kElemBytes>
__global__ __launch_bounds__(256) void kv_store_kernel(
    const uint8_t* __restrict__ k, int64_t k_stride_bytes, const uint8_t* __restrict__ v,
    int64_t v_stride_bytes, uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache,
    const int32_t* __restrict__ slots, int64_t num_chunks, int num_kv_heads, FastDiv bdiv) {
  constexpr int kRowBytes = kHeadDim * kElemBytes;
  constexpr int kChunksPerRow = kRowBytes / 16;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < num_chunks; i += stride) {
    const int64_t row = i / kChunksPerRow;  // (token, kv head)
    const int c = (int)(i % kChunksPerRow);
    const int64_t t = row / num_kv_heads;
    const int g = (int)(row % num_kv_heads);
    const int32_t s = slots[t];
    if (s < 0) continue;
    const uint32_t p = bdiv.div((uint32_t)s);  // block, row of the slot
    const int o = s - (int)(p * bdiv.d);
    const int64_t dst = (((int64_t)p * num_kv_heads + g) * bdiv.d + o) * kRowBytes + c * 16;
    const int64_t src_off = (int64_t)g * kRowBytes + c * 16;
    const u32x4 kv = *reinterpret_cast<const u32x4*>(k + t * k_stride_bytes + src_off);
    const u32x4 vv = *reinterpret_cast<const u32x4*>(v + t * v_stride_bytes + src_off);
    *reinterpret_cast<u32x4*>(k_cache + dst) = kv;
    *reinterpret_cast<u32x4*>(v_cache + dst) = vv;
  }
}

hipError_t launch_kv_store(int elem_bytes, const void* k, int64_t k_stride, const void* v,
                           int64_t v_stride, void* k_cache, void* v_cache, const int32_t* slots,
                           int num_tokens, int num_kv_heads, int block_size,
                           hipStream_t stream) {
  const int64_t chunks_per_row = (int64_t)kHeadDim * elem_bytes / 16;
  const int64_t num_chunks = (int64_t)num_tokens * num_kv_heads * chunks_per_row;
  const int threads = 256;
  int64_t blocks = (num_chunks + threads - 1) / threads;
  const int64_t max_blocks = 256 * 64;  // grid-stride beyond this
  if (blocks > max_blocks) blocks = max_blocks;
  const int64_t ksb = k_stride * elem_bytes, vsb = v_stride * elem_bytes;
  const FastDiv bdiv((uint32_t)block_size);
  if (elem_bytes == 2) {
    hipLaunchKernelGGL(kv_store_kernel<2>, dim3((unsigned)blocks), dim3(threads), 0, stream,
                       (const uint8_t*)k, ksb, (const uint8_t*)v, vsb, (uint8_t*)k_cache,
                       (uint8_t*)v_cache, slots, num_chunks, num_kv_heads, bdiv);
  } else {
    hipLaunchKernelGGL(kv_store_kernel<4>, dim3((unsigned)blocks), dim3(threads), 0, stream,
                       (const uint8_t*)k, ksb, (const uint8_t*)v, vsb, (uint8_t*)k_cache,
                       (uint8_t*)v_cache, slots, num_chunks, num_kv_heads, bdiv);
  }
  return hipGetLastError();
}

}  // namespace pkv
