// Internal launch interface between the C ABI (api.hip) and the kernels.
// Argument structs are passed to kernels by value; all pointers are device
// pointers already validated on the host.
#pragma once

#include "common.h"

namespace pa {

struct KvWriteArgs {
  const u32x4* k;        // [T, H_kv, d] as 16-byte chunks
  const u32x4* v;
  u32x4* k_cache;        // [NB, H_kv, bs, d] as 16-byte chunks
  u32x4* v_cache;
  const int32_t* slot_mapping;
  int num_tokens;
  int num_kv_heads;
  int head_chunks;       // d * sizeof(T) / 16
  int row_chunks;        // H_kv * head_chunks
  int block_size;
  int64_t num_slots;     // NB * bs
};

// paged_kv_write into E4M3 pools: 16 codes (one 16-byte chunk) per thread.
struct KvWriteFp8Args {
  const void* k;         // [T, H_kv, d] bf16 or f32
  const void* v;
  u32x4* k_cache;        // [NB, H_kv, bs, d] E4M3 codes as 16-byte chunks
  u32x4* v_cache;
  const int32_t* slot_mapping;
  const float* k_scale;  // device scalars
  const float* v_scale;
  int num_tokens;
  int num_kv_heads;
  int head_chunks;       // d / 16
  int row_chunks;        // H_kv * head_chunks
  int block_size;
  int64_t num_slots;
};

// RoPE fused into the cache write (rope.hip).
struct RopeWriteArgs {
  void* q;                     // [T, H_q, d], rotated in place
  void* k;                     // [T, H_kv, d], rotated in place
  const void* v;               // [T, H_kv, d]
  u32x4* k_cache;              // [NB, H_kv, bs, d] as 16-byte chunks
  u32x4* v_cache;
  const int32_t* slot_mapping; // [T]
  const int32_t* positions;    // [T]
  const float* cos_sin;        // [max_positions, rot_dim]: cos then sin
  int num_tokens;
  int num_q_heads;
  int num_kv_heads;
  int head_chunks;             // d * sizeof(T) / 16
  int pair_chunks;             // rot_dim / 2 * sizeof(T) / 16
  int rot_dim;
  int block_size;
  int max_positions;
  int64_t num_slots;
};

struct DecodeArgs {
  void* out;             // [B, H_q, d] (T)        when partition_size == 0
  float* lse;            // [B, H_q]               when partition_size == 0
  float* part_out;       // [B, H_q, P, d]          when partition_size > 0
  float* part_lse;       // [B, H_q, P]
  const void* q;         // [B, H_q, d]
  const void* k_cache;   // [NB, H_kv, bs, d]
  const void* v_cache;
  const int32_t* block_tables;  // [B, max_blocks_per_seq]
  const int32_t* context_lens;  // [B]
  int num_seqs;
  int num_q_heads;
  int num_kv_heads;
  int block_size;
  int max_blocks_per_seq;
  int num_blocks;
  int partition_size;    // 0 = single pass
  int num_partitions;    // partition dimension of part_* (1 when single pass)
  int max_context_len;
  float scale_log2;      // scale * log2(e)
  int flat_units;        // split-KV MFMA kernel: 1-D grid of balanced work units
  int window;            // sliding window in keys (0 = none)
  const float* k_scale;  // E4M3 pools only: device scalars, value = code * scale
  const float* v_scale;
  const void* k_new;     // append: [B, H_kv, d] K/V of the token at position ctx-1 (T),
  const void* v_new;     //   stored into the pool by the kernel before it is read; else null
  int pack_shared;       // split bf16 MFMA kernel: pack sequences that share a partition's blocks
};

struct ReduceArgs {
  void* out;
  float* lse;
  const float* part_out;
  const float* part_lse;
  const int32_t* context_lens;
  int num_seqs;
  int num_q_heads;
  int head_dim;
  int partition_size;
  int max_partitions;
  int window;            // sliding window of keys (0 = none): merge from its first partition
};

struct PrefillArgs {
  void* out;             // [T, H_q, d]
  float* lse;            // [T, H_q]
  const void* q;         // [T, H_q, d]
  const void* k;         // varlen: [T, H_kv, d]; paged: k_cache [NB, H_kv, bs, d]
  const void* v;
  const int32_t* cu_seqlens;   // query rows (and varlen keys) per sequence, [S+1]
  int num_seqs;
  int total_tokens;      // query rows
  int max_seqlen;        // longest query run
  int num_q_heads;
  int num_kv_heads;
  float scale_log2;
  // paged prefill only (block_tables == nullptr for the varlen call)
  const int32_t* block_tables;  // [S, max_blocks_per_seq]
  const int32_t* context_lens;  // [S] cached positions, the chunk included
  int block_size;
  int max_blocks_per_seq;
  int num_blocks;
  int max_context_len;
  int window;                   // sliding window in keys (0 = none)
};

enum class DType { F32 = 0, BF16 = 1 };

hipError_t launch_kv_write(const KvWriteArgs& a, hipStream_t stream);
hipError_t launch_kv_write_fp8(const KvWriteFp8Args& a, DType src, hipStream_t stream);
hipError_t launch_decode_fp8(const DecodeArgs& a, int head_dim, hipStream_t stream);
hipError_t launch_rope_cos_sin(float* table, int max_positions, int rot_dim, double base, hipStream_t stream);
hipError_t launch_rope_kv_write(const RopeWriteArgs& a, DType dt, hipStream_t stream);

// Returns hipErrorNotSupported when no kernel instance covers the shape.
hipError_t launch_decode(const DecodeArgs& a, DType dt, int head_dim, hipStream_t stream);
hipError_t launch_reduce(const ReduceArgs& a, DType dt, hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs& a, DType dt, int head_dim, hipStream_t stream);

// The vector-ALU kernels alone (also the path for shapes without an MFMA kernel).
hipError_t launch_decode_generic(const DecodeArgs& a, DType dt, int head_dim, hipStream_t stream);
hipError_t launch_prefill_generic(const PrefillArgs& a, DType dt, int head_dim, hipStream_t stream);
// The paged stream probe (stream.hip): decode's work units and tiles, read and
// folded into XOR checksums [B, H_kv, P]; LDS-DMA ring of `depth` slots, or
// `depth` tiles of register loads at a time.
hipError_t launch_stream(const DecodeArgs& a, uint32_t* sums, int depth, bool dma, hipStream_t stream);
hipError_t launch_contiguous_read(const void* src, uint64_t bytes, int waves, int depth, uint32_t* sums,
                                  hipStream_t stream);
// Paged prefill: the same kernels with keys read through the block table.
hipError_t launch_paged_prefill(const PrefillArgs& a, DType dt, int head_dim, hipStream_t stream);
hipError_t launch_paged_prefill_generic(const PrefillArgs& a, DType dt, int head_dim, hipStream_t stream);

}  // namespace pa
