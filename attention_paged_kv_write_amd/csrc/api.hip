// C ABI of the paged-attention library: argument validation, kernel choice and
// launch on the caller's stream.  No allocation, no synchronisation, no host
// read of device memory.  The declarations and their contracts are in
// include/paged_attn.h.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "kernels.h"
#include "paged_attn.h"

// The scratch array of paged_attention_decode_noalloc (see scratch_address).
static __device__ __attribute__((aligned(256))) unsigned char scratch[size_t(32) << 20];

namespace {

thread_local std::string g_last_error;
int g_force_vector_path = 0;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return PA_OK;
}

int launch_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  if (e == hipErrorNotSupported) return fail(PA_ERR_UNSUPPORTED, "%s: no kernel for these arguments", what);
  return fail(PA_ERR_LAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
}

bool dtype_ok(pa_dtype d) { return d == PA_F32 || d == PA_BF16; }
int esize(pa_dtype d) { return d == PA_BF16 ? 2 : 4; }
bool group_ok(int G) { return G == 1 || G == 2 || G == 4 || G == 8; }
// Partition dimension of a split decode's partials.
int split_parts(int max_context_len, int partition_size) {
  return max_context_len > 0 ? (max_context_len + partition_size - 1) / partition_size : 1;
}

// Scratch of paged_attention_decode_noalloc: the split partials live in this
// file-scope device array, one copy per GPU, held until the process ends.  Host
// code never passes the array's name (on the host it is only a stand-in): it
// takes the address hipGetSymbolAddress gives for the current device, once per
// device, and passes that.
constexpr size_t kScratchBytes = size_t(32) << 20;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address (looked up on its first use there).
int scratch_address(const char* fn, void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(PA_ERR_LAUNCH, "%s: no current device (%s)", fn, hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(PA_ERR_LAUNCH, "%s: scratch address on device %d: %s", fn, dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return PA_OK;
}

// Host-side checks of a decode call (everything but the output pointers);
// PA_OK means the launch may proceed (num_seqs may still be 0: nothing to do).
int decode_check(const char* fn, const void* q, const void* k_cache, const void* v_cache,
                 const int32_t* block_tables, const int32_t* context_lens, int num_seqs, int num_q_heads,
                 int num_kv_heads, int head_dim, int block_size, int max_blocks_per_seq, int num_blocks,
                 int partition_size, int max_context_len, float scale, int window, pa_dtype dtype, bool kv8,
                 const float* k_scale, const float* v_scale) {
  if (window < 0) return fail(PA_ERR_INVALID_ARG, "%s: window < 0", fn);
  if (!dtype_ok(dtype)) return fail(PA_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dtype);
  if (num_seqs < 0) return fail(PA_ERR_INVALID_ARG, "%s: num_seqs < 0", fn);
  if (num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      max_blocks_per_seq <= 0 || num_blocks <= 0)
    return fail(PA_ERR_INVALID_ARG, "%s: non-positive size", fn);
  if (num_q_heads % num_kv_heads != 0)
    return fail(PA_ERR_INVALID_ARG, "%s: num_q_heads %% num_kv_heads != 0", fn);
  if (max_context_len < 0) return fail(PA_ERR_INVALID_ARG, "%s: max_context_len < 0", fn);
  if (static_cast<int64_t>(max_context_len) > static_cast<int64_t>(max_blocks_per_seq) * block_size)
    return fail(PA_ERR_INVALID_ARG, "%s: max_context_len > max_blocks_per_seq * block_size", fn);
  if (partition_size < 0 || (partition_size > 0 && partition_size % block_size != 0))
    return fail(PA_ERR_INVALID_ARG, "%s: partition_size must be 0 or a multiple of block_size", fn);
  if (!std::isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "%s: scale is not finite", fn);
  if (num_seqs > 65535) return fail(PA_ERR_UNSUPPORTED, "%s: num_seqs > 65535", fn);
  const int G = num_q_heads / num_kv_heads;
  if (kv8) {
    if (dtype != PA_BF16 || head_dim != 128)
      return fail(PA_ERR_UNSUPPORTED, "%s: bf16 queries with head_dim 128 only", fn);
    if (!(block_size == 16 || block_size == 32 || block_size == 64))
      return fail(PA_ERR_UNSUPPORTED, "%s: block_size %d", fn, block_size);
  } else {
    if (head_dim != 64 && head_dim != 128) return fail(PA_ERR_UNSUPPORTED, "%s: head_dim %d", fn, head_dim);
    if (!(block_size == 8 || block_size == 16 || block_size == 32 || block_size == 64))
      return fail(PA_ERR_UNSUPPORTED, "%s: block_size %d", fn, block_size);
  }
  if (!group_ok(G)) return fail(PA_ERR_UNSUPPORTED, "%s: GQA group size %d", fn, G);
  if (partition_size > 0 && split_parts(max_context_len, partition_size) > 65535)
    return fail(PA_ERR_UNSUPPORTED, "%s: more than 65535 partitions", fn);
  if (num_seqs == 0) return ok();
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens)
    return fail(PA_ERR_INVALID_ARG, "%s: null input pointer", fn);
  if (kv8 && (!k_scale || !v_scale)) return fail(PA_ERR_INVALID_ARG, "%s: null k_scale/v_scale", fn);
  return PA_OK;
}

// Validation, arguments and launch shared by the decode entry points: plain or
// sliding window, bf16/f32 or E4M3 pools (kv8, with device-side scales), and
// with or without the new token's K/V (k_new, v_new) appended by the kernel.
int decode_call(const char* fn, void* out, float* lse, float* part_out, float* part_lse, const void* q,
                const void* k_new, const void* v_new, const void* k_cache, const void* v_cache,
                const int32_t* block_tables, const int32_t* context_lens, int num_seqs, int num_q_heads,
                int num_kv_heads, int head_dim, int block_size, int max_blocks_per_seq, int num_blocks,
                int partition_size, int max_context_len, float scale, int window, pa_dtype dtype, bool kv8,
                const float* k_scale, const float* v_scale, void* stream) {
  const int rc = decode_check(fn, q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_q_heads,
                              num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, partition_size,
                              max_context_len, scale, window, dtype, kv8, k_scale, v_scale);
  if (rc != PA_OK || num_seqs == 0) return rc;
  int num_parts = 1;
  if (partition_size > 0) {
    if (!part_out || !part_lse) return fail(PA_ERR_INVALID_ARG, "%s: null part_out/part_lse", fn);
    num_parts = split_parts(max_context_len, partition_size);
  } else if (!out || !lse) {
    return fail(PA_ERR_INVALID_ARG, "%s: null out/lse", fn);
  }
  pa::DecodeArgs a;
  a.out = out;
  a.lse = lse;
  a.part_out = part_out;
  a.part_lse = part_lse;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.block_size = block_size;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.partition_size = partition_size;
  a.num_partitions = num_parts;
  a.max_context_len = max_context_len;
  a.scale_log2 = scale * pa::kLog2e;
  a.flat_units = 0;
  a.window = window;
  a.k_scale = kv8 ? k_scale : nullptr;
  a.v_scale = kv8 ? v_scale : nullptr;
  a.k_new = k_new;
  a.v_new = v_new;
  a.pack_shared = 0;   // the launcher decides
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (kv8) {
    e = pa::launch_decode_fp8(a, head_dim, s);
  } else {
    const pa::DType dt = dtype == PA_BF16 ? pa::DType::BF16 : pa::DType::F32;
    e = g_force_vector_path ? pa::launch_decode_generic(a, dt, head_dim, s) : pa::launch_decode(a, dt, head_dim, s);
  }
  return launch_status(e, fn);
}

}  // namespace

extern "C" {

int pa_abi_version(void) { return 1; }

#ifndef PA_BUILD_ID
#define PA_BUILD_ID "unknown"
#endif
const char* pa_build_id(void) { return PA_BUILD_ID; }

const char* pa_last_error(void) { return g_last_error.c_str(); }

int pa_set_option(int option, int value) {
  if (option == PA_OPT_FORCE_VECTOR_PATH) {
    g_force_vector_path = value != 0;
    return ok();
  }
  return fail(PA_ERR_INVALID_ARG, "pa_set_option: unknown option %d", option);
}

int paged_kv_write(const void* k, const void* v, void* k_cache, void* v_cache,
                   const int32_t* slot_mapping, int num_tokens, int num_kv_heads, int head_dim,
                   int block_size, int num_blocks, pa_dtype dtype, void* stream) {
  if (num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "paged_kv_write: num_tokens < 0");
  if (!dtype_ok(dtype)) return fail(PA_ERR_INVALID_ARG, "paged_kv_write: unknown dtype %d", (int)dtype);
  if (num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return fail(PA_ERR_INVALID_ARG, "paged_kv_write: non-positive size");
  if (static_cast<int64_t>(num_blocks) * block_size > INT32_MAX)
    return fail(PA_ERR_INVALID_ARG, "paged_kv_write: num_blocks * block_size exceeds int32 slots");
  if ((static_cast<int64_t>(head_dim) * esize(dtype)) % 16 != 0)
    return fail(PA_ERR_UNSUPPORTED, "paged_kv_write: head_dim * sizeof(dtype) must be a multiple of 16");
  if (num_tokens == 0) return ok();
  if (!k || !v || !k_cache || !v_cache || !slot_mapping)
    return fail(PA_ERR_INVALID_ARG, "paged_kv_write: null pointer");
  pa::KvWriteArgs a;
  a.k = static_cast<const pa::u32x4*>(k);
  a.v = static_cast<const pa::u32x4*>(v);
  a.k_cache = static_cast<pa::u32x4*>(k_cache);
  a.v_cache = static_cast<pa::u32x4*>(v_cache);
  a.slot_mapping = slot_mapping;
  a.num_tokens = num_tokens;
  a.num_kv_heads = num_kv_heads;
  a.head_chunks = head_dim * esize(dtype) / 16;
  a.row_chunks = num_kv_heads * a.head_chunks;
  a.block_size = block_size;
  a.num_slots = static_cast<int64_t>(num_blocks) * block_size;
  return launch_status(pa::launch_kv_write(a, static_cast<hipStream_t>(stream)), "paged_kv_write");
}

int paged_kv_write_fp8(const void* k, const void* v, void* k_cache, void* v_cache,
                       const int32_t* slot_mapping, int num_tokens, int num_kv_heads, int head_dim,
                       int block_size, int num_blocks, const float* k_scale, const float* v_scale,
                       pa_dtype dtype, void* stream) {
  const char* fn = "paged_kv_write_fp8";
  if (num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "%s: num_tokens < 0", fn);
  if (!dtype_ok(dtype)) return fail(PA_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dtype);
  if (num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return fail(PA_ERR_INVALID_ARG, "%s: non-positive size", fn);
  if (static_cast<int64_t>(num_blocks) * block_size > INT32_MAX)
    return fail(PA_ERR_INVALID_ARG, "%s: num_blocks * block_size exceeds int32 slots", fn);
  if (head_dim % 16 != 0) return fail(PA_ERR_UNSUPPORTED, "%s: head_dim must be a multiple of 16", fn);
  if (num_tokens == 0) return ok();
  if (!k || !v || !k_cache || !v_cache || !slot_mapping || !k_scale || !v_scale)
    return fail(PA_ERR_INVALID_ARG, "%s: null pointer", fn);
  pa::KvWriteFp8Args a;
  a.k = k;
  a.v = v;
  a.k_cache = static_cast<pa::u32x4*>(k_cache);
  a.v_cache = static_cast<pa::u32x4*>(v_cache);
  a.slot_mapping = slot_mapping;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.num_tokens = num_tokens;
  a.num_kv_heads = num_kv_heads;
  a.head_chunks = head_dim / 16;
  a.row_chunks = num_kv_heads * a.head_chunks;
  a.block_size = block_size;
  a.num_slots = static_cast<int64_t>(num_blocks) * block_size;
  const pa::DType dt = dtype == PA_BF16 ? pa::DType::BF16 : pa::DType::F32;
  return launch_status(pa::launch_kv_write_fp8(a, dt, static_cast<hipStream_t>(stream)), fn);
}

int rope_cos_sin_cache(float* cos_sin, int max_positions, int rot_dim, double base, void* stream) {
  const char* fn = "rope_cos_sin_cache";
  if (max_positions < 0) return fail(PA_ERR_INVALID_ARG, "%s: max_positions < 0", fn);
  if (rot_dim <= 0 || rot_dim % 2 != 0) return fail(PA_ERR_INVALID_ARG, "%s: rot_dim must be even and positive", fn);
  if (!(base > 1.0) || !std::isfinite(base)) return fail(PA_ERR_INVALID_ARG, "%s: base must be finite and > 1", fn);
  if (static_cast<int64_t>(max_positions) * rot_dim > INT32_MAX)
    return fail(PA_ERR_UNSUPPORTED, "%s: table too large", fn);
  if (max_positions == 0) return ok();
  if (!cos_sin) return fail(PA_ERR_INVALID_ARG, "%s: null pointer", fn);
  return launch_status(pa::launch_rope_cos_sin(cos_sin, max_positions, rot_dim, base,
                                               static_cast<hipStream_t>(stream)), fn);
}

int paged_kv_write_rope(void* q, void* k, const void* v, void* k_cache, void* v_cache,
                        const int32_t* slot_mapping, const int32_t* positions, const float* cos_sin,
                        int num_tokens, int num_q_heads, int num_kv_heads, int head_dim, int rot_dim,
                        int block_size, int num_blocks, int max_positions, pa_dtype dtype, void* stream) {
  const char* fn = "paged_kv_write_rope";
  if (num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "%s: num_tokens < 0", fn);
  if (!dtype_ok(dtype)) return fail(PA_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dtype);
  if (num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0 ||
      max_positions <= 0)
    return fail(PA_ERR_INVALID_ARG, "%s: non-positive size", fn);
  if (rot_dim <= 0 || rot_dim % 2 != 0 || rot_dim > head_dim)
    return fail(PA_ERR_INVALID_ARG, "%s: rot_dim must be even, positive and <= head_dim", fn);
  if (static_cast<int64_t>(num_blocks) * block_size > INT32_MAX)
    return fail(PA_ERR_INVALID_ARG, "%s: num_blocks * block_size exceeds int32 slots", fn);
  const int es = esize(dtype);
  if ((static_cast<int64_t>(head_dim) * es) % 16 != 0 || (static_cast<int64_t>(rot_dim / 2) * es) % 16 != 0)
    return fail(PA_ERR_UNSUPPORTED, "%s: head_dim and rot_dim/2 must fill whole 16-byte chunks", fn);
  if (num_tokens == 0) return ok();
  if (!q || !k || !v || !k_cache || !v_cache || !slot_mapping || !positions || !cos_sin)
    return fail(PA_ERR_INVALID_ARG, "%s: null pointer", fn);
  pa::RopeWriteArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.k_cache = static_cast<pa::u32x4*>(k_cache);
  a.v_cache = static_cast<pa::u32x4*>(v_cache);
  a.slot_mapping = slot_mapping;
  a.positions = positions;
  a.cos_sin = cos_sin;
  a.num_tokens = num_tokens;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_chunks = head_dim * es / 16;
  a.pair_chunks = rot_dim / 2 * es / 16;
  a.rot_dim = rot_dim;
  a.block_size = block_size;
  a.max_positions = max_positions;
  a.num_slots = static_cast<int64_t>(num_blocks) * block_size;
  const pa::DType dt = dtype == PA_BF16 ? pa::DType::BF16 : pa::DType::F32;
  return launch_status(pa::launch_rope_kv_write(a, dt, static_cast<hipStream_t>(stream)), fn);
}

int paged_attention_decode(void* out, float* lse, float* part_out, float* part_lse, const void* q,
                           const void* k_cache, const void* v_cache, const int32_t* block_tables,
                           const int32_t* context_lens, int num_seqs, int num_q_heads,
                           int num_kv_heads, int head_dim, int block_size, int max_blocks_per_seq,
                           int num_blocks, int partition_size, int max_context_len, float scale,
                           pa_dtype dtype, void* stream) {
  return paged_attention_decode_window(out, lse, part_out, part_lse, q, k_cache, v_cache, block_tables,
                                       context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                       block_size, max_blocks_per_seq, num_blocks, partition_size,
                                       max_context_len, scale, 0, dtype, stream);
}

int paged_attention_decode_window(void* out, float* lse, float* part_out, float* part_lse, const void* q,
                                  const void* k_cache, const void* v_cache, const int32_t* block_tables,
                                  const int32_t* context_lens, int num_seqs, int num_q_heads,
                                  int num_kv_heads, int head_dim, int block_size, int max_blocks_per_seq,
                                  int num_blocks, int partition_size, int max_context_len, float scale,
                                  int window, pa_dtype dtype, void* stream) {
  return decode_call("paged_attention_decode", out, lse, part_out, part_lse, q, nullptr, nullptr, k_cache,
                     v_cache, block_tables, context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                     block_size, max_blocks_per_seq, num_blocks, partition_size, max_context_len, scale, window,
                     dtype, false, nullptr, nullptr, stream);
}

int paged_attention_decode_fp8(void* out, float* lse, float* part_out, float* part_lse, const void* q,
                               const void* k_cache, const void* v_cache, const int32_t* block_tables,
                               const int32_t* context_lens, int num_seqs, int num_q_heads, int num_kv_heads,
                               int head_dim, int block_size, int max_blocks_per_seq, int num_blocks,
                               int partition_size, int max_context_len, float scale, const float* k_scale,
                               const float* v_scale, int window, pa_dtype dtype, void* stream) {
  return decode_call("paged_attention_decode_fp8", out, lse, part_out, part_lse, q, nullptr, nullptr, k_cache,
                     v_cache, block_tables, context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                     block_size, max_blocks_per_seq, num_blocks, partition_size, max_context_len, scale, window,
                     dtype, true, k_scale, v_scale, stream);
}

int paged_attention_decode_append(void* out, float* lse, float* part_out, float* part_lse, const void* q,
                                  const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                                  const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                                  int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                                  int max_blocks_per_seq, int num_blocks, int partition_size, int max_context_len,
                                  float scale, int window, pa_dtype dtype, void* stream) {
  const char* fn = "paged_attention_decode_append";
  if (num_seqs > 0 && (!k_new || !v_new)) return fail(PA_ERR_INVALID_ARG, "%s: null k_new/v_new", fn);
  return decode_call(fn, out, lse, part_out, part_lse, q, k_new, v_new, k_cache, v_cache, block_tables,
                     context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                     num_blocks, partition_size, max_context_len, scale, window, dtype, false, nullptr, nullptr,
                     stream);
}

int paged_attention_decode_append_fp8(void* out, float* lse, float* part_out, float* part_lse, const void* q,
                                      const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                                      const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                                      int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                                      int max_blocks_per_seq, int num_blocks, int partition_size,
                                      int max_context_len, float scale, const float* k_scale, const float* v_scale,
                                      int window, pa_dtype dtype, void* stream) {
  const char* fn = "paged_attention_decode_append_fp8";
  if (num_seqs > 0 && (!k_new || !v_new)) return fail(PA_ERR_INVALID_ARG, "%s: null k_new/v_new", fn);
  return decode_call(fn, out, lse, part_out, part_lse, q, k_new, v_new, k_cache, v_cache, block_tables,
                     context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                     num_blocks, partition_size, max_context_len, scale, window, dtype, true, k_scale, v_scale,
                     stream);
}

int paged_attention_decode_noalloc(void* out, float* lse, const void* q, const void* k_cache, const void* v_cache,
                                   const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                                   int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                                   int max_blocks_per_seq, int num_blocks, int partition_size, int max_context_len,
                                   float scale, int window, pa_dtype dtype, void* stream) {
  const char* fn = "paged_attention_decode_noalloc";
  if (partition_size <= 0) return fail(PA_ERR_INVALID_ARG, "%s: partition_size must be > 0", fn);
  int rc = decode_check(fn, q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_q_heads, num_kv_heads,
                        head_dim, block_size, max_blocks_per_seq, num_blocks, partition_size, max_context_len,
                        scale, window, dtype, false, nullptr, nullptr);
  if (rc != PA_OK) return rc;
  const int P = split_parts(max_context_len, partition_size);
  const uint64_t rows = static_cast<uint64_t>(num_seqs) * num_q_heads * P;
  const uint64_t out_bytes = (rows * head_dim * 4 + 255) / 256 * 256;
  static_assert(sizeof(scratch) == kScratchBytes, "scratch size");
  if (out_bytes + rows * 4 > kScratchBytes)
    return fail(PA_ERR_INVALID_ARG,
                "%s: partials need %llu bytes (num_seqs * num_q_heads * partitions * (head_dim + 1) * 4), "
                "more than the %zu-byte scratch",
                fn, static_cast<unsigned long long>(out_bytes + rows * 4), kScratchBytes);
  if (num_seqs == 0) return ok();
  if (!out || !lse) return fail(PA_ERR_INVALID_ARG, "%s: null out/lse", fn);
  void* base = nullptr;
  rc = scratch_address(fn, &base);
  if (rc != PA_OK) return rc;
  float* part_out = static_cast<float*>(base);
  float* part_lse = reinterpret_cast<float*>(static_cast<unsigned char*>(base) + out_bytes);
  rc = decode_call(fn, nullptr, nullptr, part_out, part_lse, q, nullptr, nullptr, k_cache, v_cache, block_tables,
                   context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                   num_blocks, partition_size, max_context_len, scale, window, dtype, false, nullptr, nullptr,
                   stream);
  if (rc != PA_OK) return rc;
  return paged_attention_reduce_window(out, lse, part_out, part_lse, context_lens, num_seqs, num_q_heads, head_dim,
                                       partition_size, P, window, dtype, stream);
}

int paged_attention_reduce(void* out, float* lse, const float* part_out, const float* part_lse,
                           const int32_t* context_lens, int num_seqs, int num_q_heads, int head_dim,
                           int partition_size, int max_partitions, pa_dtype dtype, void* stream) {
  return paged_attention_reduce_window(out, lse, part_out, part_lse, context_lens, num_seqs, num_q_heads,
                                       head_dim, partition_size, max_partitions, 0, dtype, stream);
}

int paged_kv_stream_read(uint32_t* checksums, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* context_lens, int num_seqs, int num_kv_heads,
                         int head_dim, int block_size, int max_blocks_per_seq, int num_blocks, int partition_size,
                         int max_context_len, int mode, int depth, pa_dtype dtype, void* stream) {
  const char* fn = "paged_kv_stream_read";
  if (!dtype_ok(dtype)) return fail(PA_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dtype);
  if (num_seqs < 0) return fail(PA_ERR_INVALID_ARG, "%s: num_seqs < 0", fn);
  if (num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || max_blocks_per_seq <= 0 || num_blocks <= 0 ||
      partition_size <= 0)
    return fail(PA_ERR_INVALID_ARG, "%s: non-positive size", fn);
  if (max_context_len < 0) return fail(PA_ERR_INVALID_ARG, "%s: max_context_len < 0", fn);
  if (static_cast<int64_t>(max_context_len) > static_cast<int64_t>(max_blocks_per_seq) * block_size)
    return fail(PA_ERR_INVALID_ARG, "%s: max_context_len > max_blocks_per_seq * block_size", fn);
  if (partition_size % block_size != 0)
    return fail(PA_ERR_INVALID_ARG, "%s: partition_size must be a multiple of block_size", fn);
  if (mode != PA_STREAM_LDS_DMA && mode != PA_STREAM_REGISTERS)
    return fail(PA_ERR_INVALID_ARG, "%s: unknown mode %d", fn, mode);
  if (dtype != PA_BF16 || head_dim != 128) return fail(PA_ERR_UNSUPPORTED, "%s: bf16 head_dim 128 only", fn);
  if (!(block_size == 16 || block_size == 32 || block_size == 64))
    return fail(PA_ERR_UNSUPPORTED, "%s: block_size %d", fn, block_size);
  if (num_seqs > 65535) return fail(PA_ERR_UNSUPPORTED, "%s: num_seqs > 65535", fn);
  const int num_parts = max_context_len > 0 ? (max_context_len + partition_size - 1) / partition_size : 1;
  if (num_parts > 65535) return fail(PA_ERR_UNSUPPORTED, "%s: more than 65535 partitions", fn);
  if (num_seqs == 0) return ok();
  if (!checksums || !k_cache || !v_cache || !block_tables || !context_lens)
    return fail(PA_ERR_INVALID_ARG, "%s: null pointer", fn);
  pa::DecodeArgs a = {};
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_kv_heads;
  a.num_kv_heads = num_kv_heads;
  a.block_size = block_size;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.partition_size = partition_size;
  a.num_partitions = num_parts;
  a.max_context_len = max_context_len;
  return launch_status(pa::launch_stream(a, checksums, depth, mode == PA_STREAM_LDS_DMA,
                                         static_cast<hipStream_t>(stream)), fn);
}

int pa_stream_read_contiguous(uint32_t* checksums, const void* src, uint64_t bytes, int waves, int depth,
                              void* stream) {
  const char* fn = "pa_stream_read_contiguous";
  if (bytes % 16 != 0) return fail(PA_ERR_INVALID_ARG, "%s: bytes must be a multiple of 16", fn);
  if (waves <= 0) return fail(PA_ERR_INVALID_ARG, "%s: waves must be > 0", fn);
  if (!(depth == 1 || depth == 2 || depth == 4 || depth == 8))
    return fail(PA_ERR_UNSUPPORTED, "%s: depth %d (1, 2, 4 or 8)", fn, depth);
  if (bytes == 0) return ok();
  if (!checksums || !src) return fail(PA_ERR_INVALID_ARG, "%s: null pointer", fn);
  return launch_status(pa::launch_contiguous_read(src, bytes, waves, depth, checksums,
                                                  static_cast<hipStream_t>(stream)), fn);
}

int paged_attention_reduce_window(void* out, float* lse, const float* part_out, const float* part_lse,
                                  const int32_t* context_lens, int num_seqs, int num_q_heads, int head_dim,
                                  int partition_size, int max_partitions, int window, pa_dtype dtype,
                                  void* stream) {
  const char* fn = "paged_attention_reduce";
  if (window < 0) return fail(PA_ERR_INVALID_ARG, "%s: window < 0", fn);
  if (!dtype_ok(dtype)) return fail(PA_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dtype);
  if (num_seqs < 0) return fail(PA_ERR_INVALID_ARG, "%s: num_seqs < 0", fn);
  if (num_q_heads <= 0 || head_dim <= 0 || partition_size <= 0 || max_partitions <= 0)
    return fail(PA_ERR_INVALID_ARG, "%s: non-positive size", fn);
  if (head_dim != 64 && head_dim != 128) return fail(PA_ERR_UNSUPPORTED, "%s: head_dim %d", fn, head_dim);
  if (static_cast<int64_t>(num_seqs) * num_q_heads > INT32_MAX)
    return fail(PA_ERR_UNSUPPORTED, "%s: too many rows", fn);
  if (num_seqs == 0) return ok();
  if (!out || !lse || !part_out || !part_lse || !context_lens)
    return fail(PA_ERR_INVALID_ARG, "%s: null pointer", fn);
  pa::ReduceArgs a;
  a.out = out;
  a.lse = lse;
  a.part_out = part_out;
  a.part_lse = part_lse;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.head_dim = head_dim;
  a.partition_size = partition_size;
  a.max_partitions = max_partitions;
  a.window = window;
  const pa::DType dt = dtype == PA_BF16 ? pa::DType::BF16 : pa::DType::F32;
  return launch_status(pa::launch_reduce(a, dt, static_cast<hipStream_t>(stream)), fn);
}

int varlen_causal_prefill(void* out, float* lse, const void* q, const void* k, const void* v,
                          const int32_t* cu_seqlens, int num_seqs, int total_tokens, int max_seqlen,
                          int num_q_heads, int num_kv_heads, int head_dim, float scale,
                          pa_dtype dtype, void* stream) {
  return varlen_causal_prefill_window(out, lse, q, k, v, cu_seqlens, num_seqs, total_tokens, max_seqlen,
                                      num_q_heads, num_kv_heads, head_dim, scale, 0, dtype, stream);
}

int varlen_causal_prefill_window(void* out, float* lse, const void* q, const void* k, const void* v,
                                 const int32_t* cu_seqlens, int num_seqs, int total_tokens, int max_seqlen,
                                 int num_q_heads, int num_kv_heads, int head_dim, float scale, int window,
                                 pa_dtype dtype, void* stream) {
  const char* fn = "varlen_causal_prefill";
  if (window < 0) return fail(PA_ERR_INVALID_ARG, "%s: window < 0", fn);
  if (!dtype_ok(dtype)) return fail(PA_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dtype);
  if (num_seqs < 0 || total_tokens < 0 || max_seqlen < 0)
    return fail(PA_ERR_INVALID_ARG, "%s: negative size", fn);
  if (num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0)
    return fail(PA_ERR_INVALID_ARG, "%s: non-positive size", fn);
  if (num_q_heads % num_kv_heads != 0)
    return fail(PA_ERR_INVALID_ARG, "%s: num_q_heads %% num_kv_heads != 0", fn);
  if (max_seqlen > total_tokens) return fail(PA_ERR_INVALID_ARG, "%s: max_seqlen > total_tokens", fn);
  if (!std::isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "%s: scale is not finite", fn);
  if (head_dim != 64 && head_dim != 128) return fail(PA_ERR_UNSUPPORTED, "%s: head_dim %d", fn, head_dim);
  if (!group_ok(num_q_heads / num_kv_heads))
    return fail(PA_ERR_UNSUPPORTED, "%s: GQA group size %d", fn, num_q_heads / num_kv_heads);
  if (static_cast<int64_t>(num_q_heads) * num_seqs > INT32_MAX || num_seqs > 65535)
    return fail(PA_ERR_UNSUPPORTED, "%s: too many sequences", fn);
  if (num_seqs == 0 || total_tokens == 0 || max_seqlen == 0) return ok();
  if (!out || !lse || !q || !k || !v || !cu_seqlens) return fail(PA_ERR_INVALID_ARG, "%s: null pointer", fn);
  pa::PrefillArgs a;
  a.out = out;
  a.lse = lse;
  a.q = q;
  a.k = k;
  a.v = v;
  a.cu_seqlens = cu_seqlens;
  a.num_seqs = num_seqs;
  a.total_tokens = total_tokens;
  a.max_seqlen = max_seqlen;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.scale_log2 = scale * pa::kLog2e;
  a.block_tables = nullptr;
  a.context_lens = nullptr;
  a.block_size = 0;
  a.max_blocks_per_seq = 0;
  a.num_blocks = 0;
  a.max_context_len = 0;
  a.window = window;
  const pa::DType dt = dtype == PA_BF16 ? pa::DType::BF16 : pa::DType::F32;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = g_force_vector_path ? pa::launch_prefill_generic(a, dt, head_dim, s)
                                           : pa::launch_prefill(a, dt, head_dim, s);
  return launch_status(e, fn);
}

int paged_prefill(void* out, float* lse, const void* q, const void* k_cache, const void* v_cache,
                  const int32_t* block_tables, const int32_t* cu_seqlens_q, const int32_t* context_lens,
                  int num_seqs, int total_q, int max_seqlen_q, int num_q_heads, int num_kv_heads,
                  int head_dim, int block_size, int max_blocks_per_seq, int num_blocks,
                  int max_context_len, float scale, pa_dtype dtype, void* stream) {
  return paged_prefill_window(out, lse, q, k_cache, v_cache, block_tables, cu_seqlens_q, context_lens,
                              num_seqs, total_q, max_seqlen_q, num_q_heads, num_kv_heads, head_dim,
                              block_size, max_blocks_per_seq, num_blocks, max_context_len, scale, 0,
                              dtype, stream);
}

int paged_prefill_window(void* out, float* lse, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* cu_seqlens_q,
                         const int32_t* context_lens, int num_seqs, int total_q, int max_seqlen_q,
                         int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                         int max_blocks_per_seq, int num_blocks, int max_context_len, float scale,
                         int window, pa_dtype dtype, void* stream) {
  const char* fn = "paged_prefill";
  if (window < 0) return fail(PA_ERR_INVALID_ARG, "%s: window < 0", fn);
  if (!dtype_ok(dtype)) return fail(PA_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, (int)dtype);
  if (num_seqs < 0 || total_q < 0 || max_seqlen_q < 0 || max_context_len < 0)
    return fail(PA_ERR_INVALID_ARG, "%s: negative size", fn);
  if (num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      max_blocks_per_seq <= 0 || num_blocks <= 0)
    return fail(PA_ERR_INVALID_ARG, "%s: non-positive size", fn);
  if (num_q_heads % num_kv_heads != 0)
    return fail(PA_ERR_INVALID_ARG, "%s: num_q_heads %% num_kv_heads != 0", fn);
  if (max_seqlen_q > total_q) return fail(PA_ERR_INVALID_ARG, "%s: max_seqlen_q > total_q", fn);
  if (static_cast<int64_t>(max_context_len) > static_cast<int64_t>(max_blocks_per_seq) * block_size)
    return fail(PA_ERR_INVALID_ARG, "%s: max_context_len > max_blocks_per_seq * block_size", fn);
  if (!std::isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "%s: scale is not finite", fn);
  if (head_dim != 64 && head_dim != 128) return fail(PA_ERR_UNSUPPORTED, "%s: head_dim %d", fn, head_dim);
  if (!(block_size == 8 || block_size == 16 || block_size == 32 || block_size == 64))
    return fail(PA_ERR_UNSUPPORTED, "%s: block_size %d", fn, block_size);
  if (!group_ok(num_q_heads / num_kv_heads))
    return fail(PA_ERR_UNSUPPORTED, "%s: GQA group size %d", fn, num_q_heads / num_kv_heads);
  if (static_cast<int64_t>(num_q_heads) * num_seqs > INT32_MAX || num_seqs > 65535)
    return fail(PA_ERR_UNSUPPORTED, "%s: too many sequences", fn);
  if (num_seqs == 0 || total_q == 0 || max_seqlen_q == 0) return ok();
  if (!out || !lse || !q || !k_cache || !v_cache || !block_tables || !cu_seqlens_q || !context_lens)
    return fail(PA_ERR_INVALID_ARG, "%s: null pointer", fn);
  pa::PrefillArgs a;
  a.out = out;
  a.lse = lse;
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.cu_seqlens = cu_seqlens_q;
  a.num_seqs = num_seqs;
  a.total_tokens = total_q;
  a.max_seqlen = max_seqlen_q;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.scale_log2 = scale * pa::kLog2e;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.block_size = block_size;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.max_context_len = max_context_len;
  a.window = window;
  const pa::DType dt = dtype == PA_BF16 ? pa::DType::BF16 : pa::DType::F32;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = g_force_vector_path ? pa::launch_paged_prefill_generic(a, dt, head_dim, s)
                                           : pa::launch_paged_prefill(a, dt, head_dim, s);
  return launch_status(e, fn);
}

}  // extern "C"
