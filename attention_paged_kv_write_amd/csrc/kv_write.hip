// paged_kv_write: scatter new K/V rows into the paged pools through slots.
//
// The in-place update through the block table ("LLM inference optimisation:
// KV cache to FlashAttention", section 3.1, step 2) with a slot standing for
// (physical block, offset) ("Llama 4 inference doubling (FlashAttention-3 +
// PagedAttention + vLLM)", section 3.1).  A pure copy, so the kernel is an
// HBM stream: consecutive lanes move consecutive 16-byte chunks of the same
// token, so both the load from k/v and the store into a (block, head) slab
// are contiguous runs of head_dim * sizeof(T) bytes.
#include "kernels.h"

namespace pa {

// A wave copies TPW consecutive tokens' rows, KP passes of 64 chunks each:
// the slot lookup, its block / offset split and the row bases are
// wave-uniform (scalar), lane l of pass k takes chunk 64k + l of a token's
// K-then-V chunks (so a wave's loads and stores are contiguous runs), and
// every lane issues its KP x TPW 16-byte loads before it stores them.  Waves
// are numbered token group major, pass group minor.  Large writes use 4 x 4
// (16 loads in flight per lane); small ones 1 x 1, so that a few tokens
// still spread over many CUs.
template <int TPW, int KP>
__global__ __launch_bounds__(256) void kv_write_kernel(KvWriteArgs a) {
  const int lane = threadIdx.x & 63;
  const int per_token = 2 * a.row_chunks;   // K chunks then V chunks
  const int npg = (per_token + 64 * KP - 1) / (64 * KP);   // pass groups per token group
  const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(blockIdx.x) * 4 + (threadIdx.x >> 6));
  const int grp = w / npg, pg = w - grp * npg;
  const int t0 = grp * TPW;
  if (t0 >= a.num_tokens) return;
  int64_t sbase[TPW], dbase[TPW];
  bool live[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int t = t0 + i;
    const int slot = t < a.num_tokens ? a.slot_mapping[t] : -1;
    live[i] = slot >= 0 && static_cast<int64_t>(slot) < a.num_slots;
    const int blk = live[i] ? slot / a.block_size : 0;
    const int off = live[i] ? slot - blk * a.block_size : 0;
    sbase[i] = static_cast<int64_t>(t) * a.row_chunks;
    dbase[i] = (static_cast<int64_t>(blk) * a.num_kv_heads * a.block_size + off) * a.head_chunks;
  }
  const int head_stride = a.block_size * a.head_chunks;   // chunks from one head's slab to the next
  const int c00 = pg * 64 * KP;
  u32x4 w16[KP][TPW];
  int doff[KP];
  bool isv[KP], valid[KP];
#pragma unroll
  for (int k = 0; k < KP; ++k) {
    const int c0 = c00 + 64 * k + lane;
    valid[k] = c0 < per_token;
    isv[k] = c0 >= a.row_chunks;
    const int c = isv[k] ? c0 - a.row_chunks : c0;
    const int h = c / a.head_chunks;
    doff[k] = h * head_stride + (c - h * a.head_chunks);
    const u32x4* __restrict__ in = isv[k] ? a.v : a.k;
#pragma unroll
    for (int i = 0; i < TPW; ++i)
      if (live[i] && valid[k]) w16[k][i] = __builtin_nontemporal_load(in + sbase[i] + c);
  }
#pragma unroll
  for (int k = 0; k < KP; ++k) {
    u32x4* __restrict__ pool = isv[k] ? a.v_cache : a.k_cache;
#pragma unroll
    for (int i = 0; i < TPW; ++i)
      if (live[i] && valid[k]) pool[dbase[i] + doff[k]] = w16[k][i];
  }
}

// E4M3 pools: a lane writes one 16-byte chunk of codes (16 elements of a
// row, bf16 inputs widened exactly), quantised by quantize16_e4m3.  Waves are
// laid out as in kv_write_kernel with one token and one 64-chunk pass each, so
// that every lane has its own chunk: the quantiser's arithmetic, not memory,
// bounds this kernel.
template <bool BF>
__global__ __launch_bounds__(256) void kv_write_fp8_kernel(KvWriteFp8Args a) {
  constexpr int SRC_CHUNKS = BF ? 2 : 4;   // 16 source elements: 2 (bf16) or 4 (f32) 16-byte chunks
  const int lane = threadIdx.x & 63;
  const int per_token = 2 * a.row_chunks;   // K chunks then V chunks (of codes)
  const int npass = (per_token + 63) / 64;
  const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(blockIdx.x) * 4 + (threadIdx.x >> 6));
  const int t = w / npass, pass = w - t * npass;
  if (t >= a.num_tokens) return;
  const int slot = a.slot_mapping[t];
  if (slot < 0 || static_cast<int64_t>(slot) >= a.num_slots) return;
  const int c0 = pass * 64 + lane;
  if (c0 >= per_token) return;
  const bool is_v = c0 >= a.row_chunks;
  const int c = is_v ? c0 - a.row_chunks : c0;
  const int h = c / a.head_chunks;
  const int e = c - h * a.head_chunks;
  const int blk = slot / a.block_size;
  const int off = slot - blk * a.block_size;
  const int64_t dst = ((static_cast<int64_t>(blk) * a.num_kv_heads + h) * a.block_size + off) * a.head_chunks + e;
  const u32x4* in = static_cast<const u32x4*>(is_v ? a.v : a.k) +
                    (static_cast<int64_t>(t) * a.row_chunks + c) * SRC_CHUNKS;
  u32x4 w4[SRC_CHUNKS];
#pragma unroll
  for (int i = 0; i < SRC_CHUNKS; ++i) w4[i] = __builtin_nontemporal_load(in + i);
  float x[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if constexpr (BF) {
      const uint32_t word = w4[i / 8][(i % 8) / 2];
      x[i] = (i & 1) ? bf16_hi(word) : bf16_lo(word);
    } else {
      x[i] = __uint_as_float(w4[i / 4][i % 4]);
    }
  }
  const u32x4 out = quantize16_e4m3(x, scale_rcp(is_v ? a.v_scale[0] : a.k_scale[0]));
  u32x4* pool = is_v ? a.v_cache : a.k_cache;
  pool[dst] = out;
}

hipError_t launch_kv_write_fp8(const KvWriteFp8Args& a, DType src, hipStream_t stream) {
  if (a.num_tokens == 0 || a.row_chunks == 0) return hipSuccess;
  const int64_t waves = static_cast<int64_t>(a.num_tokens) * ((2LL * a.row_chunks + 63) / 64);
  const int64_t blocks = (waves + 3) / 4;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(blocks));
  if (src == DType::BF16)
    hipLaunchKernelGGL(kv_write_fp8_kernel<true>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(kv_write_fp8_kernel<false>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_kv_write(const KvWriteArgs& a, hipStream_t stream) {
  if (a.num_tokens == 0 || a.row_chunks == 0) return hipSuccess;
  const int64_t passes = (2LL * a.row_chunks + 63) / 64;   // 64-chunk passes per token
  auto waves = [&](int tpw, int kp) {
    return (static_cast<int64_t>(a.num_tokens) + tpw - 1) / tpw * ((passes + kp - 1) / kp);
  };
  if (a.num_tokens >= 4096) {
    const int64_t blocks = (waves(4, 4) + 3) / 4;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((kv_write_kernel<4, 4>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, a);
  } else {
    const int64_t blocks = (waves(1, 1) + 3) / 4;
    hipLaunchKernelGGL((kv_write_kernel<1, 1>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace pa
