// paged_kv_write: scatter new K/V rows into the paged pools through slots.
//
// The in-place update through the block table ("LLM inference optimisation:
// KV cache to FlashAttention", section 3.1, step 2) with a slot standing for
// (physical block, offset) ("Llama 4 inference doubling (FlashAttention-3 +
// PagedAttention + vLLM)", section 3.1).  A pure copy, so the kernel is an
// HBM stream: every thread moves one 16-byte chunk of a row, consecutive
// threads move consecutive chunks of the same token, so both the load from
// k/v and the store into a (block, head) slab are contiguous runs of
// head_dim * sizeof(T) bytes.
#include "kernels.h"

namespace pa {

__global__ __launch_bounds__(256) void kv_write_kernel(KvWriteArgs a) {
  const int64_t item = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t per_token = 2LL * a.row_chunks;  // K chunks then V chunks
  if (item >= static_cast<int64_t>(a.num_tokens) * per_token) return;
  const int t = static_cast<int>(item / per_token);
  int c = static_cast<int>(item - static_cast<int64_t>(t) * per_token);
  const bool is_v = c >= a.row_chunks;
  if (is_v) c -= a.row_chunks;
  const int slot = a.slot_mapping[t];
  if (slot < 0 || static_cast<int64_t>(slot) >= a.num_slots) return;
  const int h = c / a.head_chunks;
  const int e = c - h * a.head_chunks;
  const int blk = slot / a.block_size;
  const int off = slot - blk * a.block_size;
  const int64_t dst =
      ((static_cast<int64_t>(blk) * a.num_kv_heads + h) * a.block_size + off) * a.head_chunks + e;
  const int64_t src = static_cast<int64_t>(t) * a.row_chunks + c;
  const u32x4* __restrict__ in = is_v ? a.v : a.k;
  u32x4* __restrict__ pool = is_v ? a.v_cache : a.k_cache;
  pool[dst] = __builtin_nontemporal_load(in + src);
}

hipError_t launch_kv_write(const KvWriteArgs& a, hipStream_t stream) {
  const int64_t items = static_cast<int64_t>(a.num_tokens) * 2 * a.row_chunks;
  if (items == 0) return hipSuccess;
  const int64_t blocks = (items + 255) / 256;
  hipLaunchKernelGGL(kv_write_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
