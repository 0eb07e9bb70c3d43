// Rotary position embedding fused into the cache write.
//
// "LLaMA inference performance: structure and source" (section 2.2) turns
// every query and key vector, before the product, by a position-dependent
// rotation computed from sin and cos, and points to caching the table of
// those values; its attention listing applies it as the first step.  Here
// dims i and i + r/2 of the first r dims of a head form a pair turned by the
// angle p * base^(-2i/r) at position p.
//
// rope_cos_sin_kernel fills the cached table [max_positions, r] (cos in the
// first half of a row, sin in the second) from fp64 angles, cos and sin, so
// each entry is the exact value rounded once to fp32.
//
// rope_kv_write_kernel is one HBM pass over the step's rows: a thread owns
// one 16-byte chunk of the first half of a rotated head row and the matching
// chunk of the second half, turns them in fp32 with the table, stores them
// back in place (q and k) and, for k, into the pool slot; v rows and the
// dims past r are 16-byte copies into the pool.  Consecutive threads take
// consecutive chunks of one head, so every load and store is a contiguous run.
#include "kernels.h"

namespace pa {

__global__ __launch_bounds__(256) void rope_cos_sin_kernel(float* table, int max_positions, int rot_dim,
                                                           double base) {
  const int half = rot_dim / 2;
  const int64_t item = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (item >= static_cast<int64_t>(max_positions) * half) return;
  const int p = static_cast<int>(item / half);
  const int i = static_cast<int>(item - static_cast<int64_t>(p) * half);
  const double inv_freq = pow(base, -2.0 * i / rot_dim);
  const double ang = static_cast<double>(p) * inv_freq;
  table[static_cast<int64_t>(p) * rot_dim + i] = static_cast<float>(cos(ang));
  table[static_cast<int64_t>(p) * rot_dim + half + i] = static_cast<float>(sin(ang));
}

hipError_t launch_rope_cos_sin(float* table, int max_positions, int rot_dim, double base, hipStream_t stream) {
  const int64_t items = static_cast<int64_t>(max_positions) * (rot_dim / 2);
  if (items == 0) return hipSuccess;
  hipLaunchKernelGGL(rope_cos_sin_kernel, dim3(static_cast<unsigned>((items + 255) / 256)), dim3(256), 0,
                     stream, table, max_positions, rot_dim, base);
  return hipGetLastError();
}

namespace {

constexpr int kF32PerChunk = 4;

// Elements of a 16-byte chunk as floats (bf16: 8, f32: 4).
template <bool BF>
__device__ __forceinline__ void chunk_to_f32(const u32x4& w, float* x) {
  if constexpr (BF) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16_lo(w[i]);
      x[2 * i + 1] = bf16_hi(w[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(w[i]);
  }
}

template <bool BF>
__device__ __forceinline__ u32x4 f32_to_chunk(const float* x) {
  u32x4 w;
  if constexpr (BF) {
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = __float_as_uint(x[i]);
  }
  return w;
}

}  // namespace

// Items of a token, in order: q pairs (H_q x pair_chunks), k pairs (H_kv x
// pair_chunks), k pass-through chunks (H_kv x (head_chunks - 2 pair_chunks)),
// v chunks (H_kv x head_chunks).
template <bool BF>
__global__ __launch_bounds__(256) void rope_kv_write_kernel(RopeWriteArgs a) {
  constexpr int E = BF ? 8 : 4;   // elements per 16-byte chunk
  const int PC = a.pair_chunks, HC = a.head_chunks, TC = HC - 2 * PC;
  const int nq = a.num_q_heads * PC, nk = a.num_kv_heads * PC, nt = a.num_kv_heads * TC;
  const int per_token = nq + nk + nt + a.num_kv_heads * HC;
  const int64_t item = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (item >= static_cast<int64_t>(a.num_tokens) * per_token) return;
  const int t = static_cast<int>(item / per_token);
  int c = static_cast<int>(item - static_cast<int64_t>(t) * per_token);
  const int slot = a.slot_mapping[t];
  const bool write = slot >= 0 && static_cast<int64_t>(slot) < a.num_slots;
  const int blk = write ? slot / a.block_size : 0;
  const int off = write ? slot - blk * a.block_size : 0;
  auto pool_chunk = [&](int h, int e) -> int64_t {
    return ((static_cast<int64_t>(blk) * a.num_kv_heads + h) * a.block_size + off) * HC + e;
  };

  if (c < nq + nk) {
    const bool is_q = c < nq;
    if (!is_q) c -= nq;
    const int h = c / PC, e = c - h * PC;   // first-half chunk e, second-half chunk PC + e
    const int H = is_q ? a.num_q_heads : a.num_kv_heads;
    u32x4* row = static_cast<u32x4*>(is_q ? a.q : a.k) + (static_cast<int64_t>(t) * H + h) * HC;
    const int p = clampi(a.positions[t], 0, a.max_positions - 1);   // out of range: unspecified, memory safe
    const float* cs = a.cos_sin + static_cast<int64_t>(p) * a.rot_dim + e * E;
    const int half = a.rot_dim / 2;
    float x1[E], x2[E], c8[E], s8[E];
    chunk_to_f32<BF>(row[e], x1);
    chunk_to_f32<BF>(row[PC + e], x2);
#pragma unroll
    for (int i = 0; i < E; i += kF32PerChunk) {
      const u32x4 cw = *reinterpret_cast<const u32x4*>(cs + i);
      const u32x4 sw = *reinterpret_cast<const u32x4*>(cs + half + i);
#pragma unroll
      for (int j = 0; j < kF32PerChunk; ++j) {
        c8[i + j] = __uint_as_float(cw[j]);
        s8[i + j] = __uint_as_float(sw[j]);
      }
    }
    float y1[E], y2[E];
#pragma unroll
    for (int i = 0; i < E; ++i) {
      y1[i] = x1[i] * c8[i] - x2[i] * s8[i];
      y2[i] = x2[i] * c8[i] + x1[i] * s8[i];
    }
    const u32x4 w1 = f32_to_chunk<BF>(y1), w2 = f32_to_chunk<BF>(y2);
    row[e] = w1;
    row[PC + e] = w2;
    if (!is_q && write) {
      a.k_cache[pool_chunk(h, e)] = w1;
      a.k_cache[pool_chunk(h, PC + e)] = w2;
    }
    return;
  }
  c -= nq + nk;
  if (!write) return;
  if (c < nt) {   // k dims past the rotated ones
    const int h = c / TC, e = 2 * PC + (c - h * TC);
    const u32x4* row = static_cast<const u32x4*>(a.k) + (static_cast<int64_t>(t) * a.num_kv_heads + h) * HC;
    a.k_cache[pool_chunk(h, e)] = row[e];
    return;
  }
  c -= nt;
  const int h = c / HC, e = c - h * HC;
  const u32x4* row = static_cast<const u32x4*>(a.v) + (static_cast<int64_t>(t) * a.num_kv_heads + h) * HC;
  a.v_cache[pool_chunk(h, e)] = __builtin_nontemporal_load(row + e);
}

hipError_t launch_rope_kv_write(const RopeWriteArgs& a, DType dt, hipStream_t stream) {
  const int64_t per_token = static_cast<int64_t>(a.num_q_heads) * a.pair_chunks +
                            static_cast<int64_t>(a.num_kv_heads) * (a.head_chunks - a.pair_chunks) +
                            static_cast<int64_t>(a.num_kv_heads) * a.head_chunks;
  const int64_t items = static_cast<int64_t>(a.num_tokens) * per_token;
  if (items == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((items + 255) / 256));
  if (dt == DType::BF16)
    hipLaunchKernelGGL(rope_kv_write_kernel<true>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(rope_kv_write_kernel<false>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
