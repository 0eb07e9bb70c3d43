// paged_attention_decode: one query token per sequence against its paged history.
//
// What is computed is PagedAttention decode ("PageAttention + FlashAttention
// golden combination", section 2.1; "Llama 4 inference doubling
// (FlashAttention-3 + PagedAttention + vLLM)", section 3.1): the K/V rows of
// a sequence are fetched block by block through its int32 block table, query
// heads share KV heads in groups ("LLaMA inference performance: structure and
// source", section 2.1), and the softmax is done online (running max, running
// sum, rescaled accumulator) so scores never leave registers, the IO-aware
// fusion the FlashAttention sections of those pages describe.
//
// Work units: with a partition size, one wave per (KV head, sequence,
// partition), the partial results merged by paged_attention_reduce; without,
// one workgroup of four waves per (KV head, sequence) that take the blocks
// round-robin and merge their softmax states through LDS.  The work split
// depends only on logical positions, never on physical block ids, so
// permuting the pool leaves every result bit-identical.
//
// Three kernels:
//  * decode_mfma_kernel (bf16, head_dim 128): K and V tiles of 16 tokens are
//    staged in LDS by LDS-DMA; QK^T against the whole GQA group is a chain of
//    four v_mfma_f32_16x16x32_bf16 and P.V eight v_mfma_f32_16x16x16_bf16 (see
//    the comment above the kernel).
//  * decode_fp8_kernel (E4M3 pools, head_dim 128): the same scheme over
//    32-row steps, codes converted to bf16 operands in registers, V^T read
//    straight from the code tile by transposed byte reads.
//  * decode_generic_kernel (fp32 or bf16, head_dim 64/128): vector ALU only;
//    LPT lanes share a token row, dot products reduced with DPP.
#include "kernels.h"
#include "units.h"

// Cache policy of the K/V LDS-DMA loads (each cache byte is read once).
#ifndef PA_DECODE_AUX
#define PA_DECODE_AUX 2
#endif

namespace pa {

namespace {

template <bool BF>
__device__ __forceinline__ void unpack16(const u32x4 w, float* f) {
  if constexpr (BF) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16_lo(w[i]);
      f[2 * i + 1] = bf16_hi(w[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(w[i]);
  }
}

// Final cross-wave merge of (m, l, acc) held in LDS and the store of the result.
// sm_m/sm_l: [4][G]; sm_acc: [4][G][D].  m is in log2 units.
template <bool BF, int D, int G, int W = 4>
__device__ __forceinline__ void merge_and_store(const DecodeArgs& a, int b, int g, int part,
                                                const float (*sm_m)[G], const float (*sm_l)[G],
                                                const float (*sm_acc)[G][D]) {
  for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
    const int h = idx / D;
    const int e = idx - h * D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < W; ++w) M = fmaxf(M, sm_m[w][h]);
    float o = 0.f, lse = kNegInf;
    if (M != kNegInf) {
      float L = 0.f, acc = 0.f;
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const float f = fast_exp2(sm_m[w][h] - M);
        L += f * sm_l[w][h];
        acc += f * sm_acc[w][h][e];
      }
      o = acc / L;
      lse = (M + __log2f(L)) * kLn2;
    }
    const int hq = g * G + h;
    const size_t row = static_cast<size_t>(b) * a.num_q_heads + hq;
    if (a.partition_size > 0) {
      const size_t pr = row * a.num_partitions + part;
      a.part_out[pr * D + e] = o;
      if (e == 0) a.part_lse[pr] = lse;
    } else {
      if constexpr (BF) {
        static_cast<uint16_t*>(a.out)[row * D + e] = f32_to_bf16_bits(o);
      } else {
        static_cast<float*>(a.out)[row * D + e] = o;
      }
      if (e == 0) a.lse[row] = lse;
    }
  }
}

// Empty single-pass range (ctx = 0): out = 0, lse = -inf for the group's heads.
template <bool BF, int D, int G>
__device__ __forceinline__ void store_empty(const DecodeArgs& a, int b, int g) {
  for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
    const int h = idx / D;
    const int e = idx - h * D;
    const size_t row = static_cast<size_t>(b) * a.num_q_heads + g * G + h;
    if constexpr (BF) {
      static_cast<uint16_t*>(a.out)[row * D + e] = 0;
    } else {
      static_cast<float*>(a.out)[row * D + e] = 0.f;
    }
    if (e == 0) a.lse[row] = kNegInf;
  }
}

// Append: store the new token's K and V (k_new/v_new row (b, g), the token at
// position ctx-1) into its pool slot (block `phys`, offset `off`), then wait
// until the stores have completed, so this wave's later loads of that block
// see them.  Only the wave that reads position ctx-1 calls this, and no other
// workgroup reads that row, so no wider ordering is needed.  Pool rows of
// bf16/f32 are copied chunk by chunk (lanes 0 .. RC-1 K, RC .. 2RC-1 V); E4M3
// rows take 16 elements per lane, quantised with the pool's scale.
template <int D, int ESZ, bool KV8>
__device__ __forceinline__ void append_new_token(const DecodeArgs& a, int b, int g, int phys, int off, int lane) {
  constexpr int RC = D * ESZ / 16;                      // source chunks per row
  constexpr int PRC = KV8 ? D / 16 : RC;                // pool chunks per row
  if (lane < 2 * PRC) {
    const bool is_v = lane >= PRC;
    const int c = is_v ? lane - PRC : lane;
    const u32x4* src = static_cast<const u32x4*>(is_v ? a.v_new : a.k_new) +
                       (static_cast<size_t>(b) * a.num_kv_heads + g) * RC;
    u32x4* pool = const_cast<u32x4*>(static_cast<const u32x4*>(is_v ? a.v_cache : a.k_cache));
    const size_t dst = ((static_cast<size_t>(phys) * a.num_kv_heads + g) * a.block_size + off) * PRC + c;
    if constexpr (KV8) {
      float x[16];
      const u32x4 w0 = src[2 * c], w1 = src[2 * c + 1];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[2 * i] = bf16_lo(w0[i]);
        x[2 * i + 1] = bf16_hi(w0[i]);
        x[8 + 2 * i] = bf16_lo(w1[i]);
        x[8 + 2 * i + 1] = bf16_hi(w1[i]);
      }
      pool[dst] = quantize16_e4m3(x, is_v ? a.v_scale[0] : a.k_scale[0]);
    } else {
      pool[dst] = src[c];
    }
  }
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#endif
}

// The block index of position ctx-1 if this wave of this work unit reads it
// (and an append was asked for), else -1.
__device__ __forceinline__ int append_block(const DecodeArgs& a, const Range& r, int wave, int W) {
  if (a.k_new == nullptr || r.ctx <= 0) return -1;
  const int lblk = (r.ctx - 1) / a.block_size;
  if (lblk < r.blk_lo || lblk >= r.blk_hi || (lblk - r.blk_lo) % W != wave) return -1;
  return lblk;
}

}  // namespace

// ---------------------------------------------------------------------------
// Vector-ALU kernel (any supported dtype / head_dim)
// ---------------------------------------------------------------------------
template <bool BF, int D, int G>
__global__ __launch_bounds__(256) void decode_generic_kernel(DecodeArgs a) {
  constexpr int ESZ = BF ? 2 : 4;
  constexpr int VEC = 16 / ESZ;        // elements per lane per row
  constexpr int LPT = D * ESZ / 16;    // lanes per token row
  constexpr int TPW = 64 / LPT;        // token rows per wave-wide load
  constexpr int CH = 4;                // rows per lane per online-softmax step
  constexpr int ROW_CHUNKS = D * ESZ / 16;

  __shared__ float sm_m[4][G];
  __shared__ float sm_l[4][G];
  __shared__ float sm_acc[4][G][D];

  const int g = blockIdx.x, b = blockIdx.y, part = blockIdx.z;
  const Range r = work_range(a, b, part);
  if (r.blk_lo >= r.blk_hi) {
    if (a.partition_size == 0) store_empty<BF, D, G>(a, b, g);
    return;
  }
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int rg = lane / LPT, dl = lane % LPT;
  const int BS = a.block_size;
  {
    const int lblk = append_block(a, r, wave, 4);   // the waves take blocks round-robin
    if (lblk >= 0) {
      const int phys = a.block_tables[static_cast<size_t>(b) * a.max_blocks_per_seq + lblk];
      if (phys >= 0 && phys < a.num_blocks) append_new_token<D, ESZ, false>(a, b, g, phys, (r.ctx - 1) % BS, lane);
    }
  }

  float qv[G][VEC];
  {
    const u32x4* qc = static_cast<const u32x4*>(a.q);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const size_t row = static_cast<size_t>(b) * a.num_q_heads + g * G + h;
      unpack16<BF>(qc[row * ROW_CHUNKS + dl], qv[h]);
    }
  }
  float m[G], l[G], acc[G][VEC];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kNegInf;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[h][e] = 0.f;
  }

  const u32x4* kc = static_cast<const u32x4*>(a.k_cache);
  const u32x4* vc = static_cast<const u32x4*>(a.v_cache);
  for (int blk = r.blk_lo + wave; blk < r.blk_hi; blk += 4) {
    const int phys = a.block_tables[static_cast<size_t>(b) * a.max_blocks_per_seq + blk];
    if (phys < 0 || phys >= a.num_blocks) continue;  // precondition violation: skip the block
    const size_t slab = (static_cast<size_t>(phys) * a.num_kv_heads + g) * BS * ROW_CHUNKS;
    for (int r0 = 0; r0 < BS; r0 += TPW * CH) {
      float s[CH][G];
      float vv[CH][VEC];
      bool valid[CH];
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int row = r0 + c * TPW + rg;
        valid[c] = row < BS && blk * BS + row < r.ctx && blk * BS + row >= r.lo;
        float kf[VEC];
        if (valid[c]) {
          unpack16<BF>(kc[slab + static_cast<size_t>(row) * ROW_CHUNKS + dl], kf);
          unpack16<BF>(vc[slab + static_cast<size_t>(row) * ROW_CHUNKS + dl], vv[c]);
        } else {
#pragma unroll
          for (int e = 0; e < VEC; ++e) kf[e] = vv[c][e] = 0.f;
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float t = 0.f;
#pragma unroll
          for (int e = 0; e < VEC; ++e) t = fmaf(qv[h][e], kf[e], t);
          s[c][h] = group_allreduce<LPT>(t, OpSum());
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float mx = kNegInf;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
          s[c][h] = valid[c] ? s[c][h] * a.scale_log2 : kNegInf;
          mx = fmaxf(mx, s[c][h]);
        }
        const float m_new = fmaxf(m[h], mx);
        const float ms = m_new == kNegInf ? 0.f : m_new;
        const float alpha = fast_exp2(m[h] - ms);
        m[h] = m_new;
        l[h] *= alpha;
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[h][e] *= alpha;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
          const float p = fast_exp2(s[c][h] - ms);
          l[h] += p;
#pragma unroll
          for (int e = 0; e < VEC; ++e) acc[h][e] = fmaf(p, vv[c][e], acc[h][e]);
        }
      }
    }
  }

  // merge the TPW row groups of the wave (lanes differing in bits >= log2(LPT))
#pragma unroll
  for (int step = LPT; step < 64; step *= 2) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mo = xchg_xor(m[h], step);
      const float lo = xchg_xor(l[h], step);
      const float M = fmaxf(m[h], mo);
      const float ms = M == kNegInf ? 0.f : M;
      const float f = fast_exp2(m[h] - ms), fo = fast_exp2(mo - ms);
      l[h] = l[h] * f + lo * fo;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float ao = xchg_xor(acc[h][e], step);
        acc[h][e] = acc[h][e] * f + ao * fo;
      }
      m[h] = M;
    }
  }
  if (rg == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) sm_acc[wave][h][dl * VEC + e] = acc[h][e];
      if (dl == 0) {
        sm_m[wave][h] = m[h];
        sm_l[wave][h] = l[h];
      }
    }
  }
  __syncthreads();
  merge_and_store<BF, D, G>(a, b, g, part, sm_m, sm_l, sm_acc);
}

// Read one decode tile back from its LDS ring slot: the four lane-linear
// 16-byte K reads and the eight transposed V reads, then wait for them.  The
// slot's byte offset OFF is an immediate of each read (no address arithmetic
// per tile).  Inline asm (only in the device pass: its register constraints
// mean nothing to the host compiler) so that the compiler, which cannot track
// LDS-DMA completions, adds no wait of its own for the DMA loads in flight.
template <int OFF>
__device__ __forceinline__ void lds_read_decode_tile(u32x4* kw, u32x2* vt, const uint32_t* k_addr,
                                                     const uint32_t* v_addr) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile(
      "ds_read_b128 %0, %12 offset:%24\n\t"
      "ds_read_b128 %1, %13 offset:%24\n\t"
      "ds_read_b128 %2, %14 offset:%24\n\t"
      "ds_read_b128 %3, %15 offset:%24\n\t"
      "ds_read_b64_tr_b16 %4, %16 offset:%24\n\t"
      "ds_read_b64_tr_b16 %5, %17 offset:%24\n\t"
      "ds_read_b64_tr_b16 %6, %18 offset:%24\n\t"
      "ds_read_b64_tr_b16 %7, %19 offset:%24\n\t"
      "ds_read_b64_tr_b16 %8, %20 offset:%24\n\t"
      "ds_read_b64_tr_b16 %9, %21 offset:%24\n\t"
      "ds_read_b64_tr_b16 %10, %22 offset:%24\n\t"
      "ds_read_b64_tr_b16 %11, %23 offset:%24\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(kw[0]), "=&v"(kw[1]), "=&v"(kw[2]), "=&v"(kw[3]), "=&v"(vt[0]), "=&v"(vt[1]),
        "=&v"(vt[2]), "=&v"(vt[3]), "=&v"(vt[4]), "=&v"(vt[5]), "=&v"(vt[6]), "=&v"(vt[7])
      : "v"(k_addr[0]), "v"(k_addr[1]), "v"(k_addr[2]), "v"(k_addr[3]), "v"(v_addr[0]), "v"(v_addr[1]),
        "v"(v_addr[2]), "v"(v_addr[3]), "v"(v_addr[4]), "v"(v_addr[5]), "v"(v_addr[6]), "v"(v_addr[7]),
        "i"(OFF)
      : "memory");
#else
  (void)kw; (void)vt; (void)k_addr; (void)v_addr;
#endif
}

// FP8 step: this lane's 64 K codes (two 16-byte reads per tile) and its eight
// transposed V reads (8 codes each) from its LDS ring slot (byte offset OFF),
// then wait for them (inline asm for the same reason as the bf16 tile read).
template <int OFF>
__device__ __forceinline__ void lds_read_fp8_step(u32x4* k8, u32x2* v8, const uint32_t* k_addr,
                                                  const uint32_t* v_addr) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile(
      "ds_read_b128 %0, %12 offset:%24\n\t"
      "ds_read_b128 %1, %13 offset:%24\n\t"
      "ds_read_b128 %2, %14 offset:%24\n\t"
      "ds_read_b128 %3, %15 offset:%24\n\t"
      "ds_read_b64_tr_b8 %4, %16 offset:%24\n\t"
      "ds_read_b64_tr_b8 %5, %17 offset:%24\n\t"
      "ds_read_b64_tr_b8 %6, %18 offset:%24\n\t"
      "ds_read_b64_tr_b8 %7, %19 offset:%24\n\t"
      "ds_read_b64_tr_b8 %8, %20 offset:%24\n\t"
      "ds_read_b64_tr_b8 %9, %21 offset:%24\n\t"
      "ds_read_b64_tr_b8 %10, %22 offset:%24\n\t"
      "ds_read_b64_tr_b8 %11, %23 offset:%24\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(k8[0]), "=&v"(k8[1]), "=&v"(k8[2]), "=&v"(k8[3]), "=&v"(v8[0]), "=&v"(v8[1]),
        "=&v"(v8[2]), "=&v"(v8[3]), "=&v"(v8[4]), "=&v"(v8[5]), "=&v"(v8[6]), "=&v"(v8[7])
      : "v"(k_addr[0]), "v"(k_addr[1]), "v"(k_addr[2]), "v"(k_addr[3]), "v"(v_addr[0]), "v"(v_addr[1]),
        "v"(v_addr[2]), "v"(v_addr[3]), "v"(v_addr[4]), "v"(v_addr[5]), "v"(v_addr[6]), "v"(v_addr[7]),
        "i"(OFF)
      : "memory");
#else
  (void)k8; (void)v8; (void)k_addr; (void)v_addr;
#endif
}


// Eight E4M3 codes (two dwords) -> eight bf16 (exact: every E4M3 value is a
// bf16 value), low byte first.  The convert's scale operand is 1.
__device__ __forceinline__ u32x4 e4m3x8_to_bf16(uint32_t w0, uint32_t w1) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.f, false));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.f, true));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.f, false));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.f, true));
  return r;
}


// ---------------------------------------------------------------------------
// Pieces shared by the two MFMA kernels (head_dim 128, one GQA group of G
// query heads per wave as the 16 columns of the matrix products)
// ---------------------------------------------------------------------------
// The work unit of this workgroup: KV head g, sequence b, partition part.
// W == 1 with a flat grid: the balanced unit of the id (b = -1 past the
// last unit); otherwise the grid coordinates.
struct UnitId {
  int g, b, part;
};
// Flat grid ids: head-major (id = unit * H_kv + g) puts KV head g of every
// unit on XCD id mod 8; XCD-major (XM) gives XCD x the units u = x mod 8 with
// all their KV heads (id = (u / 8) * 8 H_kv + g * 8 + u mod 8, the grid
// rounded up to a multiple of 8 H_kv), so an XCD reads every head's slab of
// the blocks it touches.  The E4M3 kernel, whose 2 KB slabs are half the
// bf16 ones, streams a little faster XCD-major (workload 8 at 512-token
// partitions, same-box A/B on three boxes: 1.4-3.8%, e.g. 28.34 +- 0.13 vs
// 28.74 +- 0.10 us over four rounds); the bf16 kernel at its 1024-token
// partitions does not (48.0-48.2 vs 47.8-47.9 us), so it stays head-major.
template <int W, bool XM = false>
__device__ __forceinline__ UnitId unit_id(const DecodeArgs& a) {
  if (W == 1 && a.flat_units) {
    const int Hkv = a.num_kv_heads;
    int ui = blockIdx.x / Hkv, gi = blockIdx.x % Hkv;
    if constexpr (XM) {
      const int r = blockIdx.x >> 3;
      gi = r % Hkv;
      ui = (r / Hkv) * 8 + (blockIdx.x & 7);
    }
    const Unit un = flat_unit(a, ui);
    if (un.b < 0) return {0, -1, 0};
    return {gi, __builtin_amdgcn_readfirstlane(un.b), __builtin_amdgcn_readfirstlane(un.part)};
  }
  return {static_cast<int>(blockIdx.x), static_cast<int>(blockIdx.y), static_cast<int>(blockIdx.z)};
}

// Column packing.  The 16 B-operand columns of the matrix products hold the G
// query heads of one sequence; with G < 16 the other columns can carry the
// heads of PK - 1 = 16/G - 1 more sequences at no extra matrix work, when
// they read the same keys.  Sequences L = b - b % PK .. L + PK - 1 form a
// pack: member L + k joins its leader's work unit for a partition when both
// see the whole partition and their block ids over it are identical (the
// blocks of a prompt shared copy-on-write, "PageAttention + FlashAttention
// golden combination", section 2.1).  The leader's unit then computes the
// partition for every member (column c16 belongs to member c16 / G) and the
// members' own units exit; a sequence that shares nothing with its leader is
// its own unit as before.  Both sides take the decision from the same table
// entries and context lengths, so it is the same on both.
struct Pack {
  int lead;          // the sequence whose unit computes this partition
  uint32_t mask;     // bit k: sequence lead + k is in the unit
  bool follower;     // this unit's partition is computed by its leader's unit
};
template <int PK, int BS>
__device__ __forceinline__ Pack pack_of(const DecodeArgs& a, int b, int part, int lane) {
  const int nblk = a.partition_size / BS;   // at most 64 (checked by the launcher)
  const int e = part * nblk + lane;
  const bool in = lane < nblk && e < a.max_blocks_per_seq;
  const int cap = min(a.max_context_len, a.max_blocks_per_seq * BS);
  const int pend = (part + 1) * a.partition_size;
  const int lead = b - b % PK;
  auto row = [&](int s) { return a.block_tables + static_cast<size_t>(s) * a.max_blocks_per_seq; };
  auto whole = [&](int s) { return clampi(a.context_lens[s], 0, cap) >= pend; };
  const int lead_id = in ? row(lead)[e] : 0;
  const bool lead_whole = whole(lead);
  auto shares = [&](int s) {
    const int id = in ? row(s)[e] : 0;
    return lead_whole && whole(s) && __builtin_amdgcn_ballot_w64(id != lead_id) == 0;
  };
  if (b != lead) return Pack{b, 1u, shares(b)};
  uint32_t mask = 1u;
#pragma unroll
  for (int k = 1; k < PK; ++k)
    if (lead + k < a.num_seqs && shares(lead + k)) mask |= 1u << k;
  return Pack{lead, mask, false};
}

// The group's queries as the B operand of the four QK^T MFMAs: column c16 is
// query head g*G + c16 % G of sequence b + c16 / G when bit c16 / G of pack is
// set, else zero; MFMA c takes 16-byte chunk 4c + j of the bf16 row, or chunk
// 4j + c when the dims run in the E4M3 kernel's permuted order.  qsign flips
// the sign bits (a negative softmax scale).
template <int G, bool PERMUTED>
__device__ __forceinline__ void load_group_queries(const DecodeArgs& a, int b, uint32_t pack, int g, int j,
                                                   int c16, uint32_t qsign, bf16x8* qf) {
  constexpr int RC = 16;   // 16-byte chunks per bf16 row of 128
  const u32x4* qc = static_cast<const u32x4*>(a.q);
  const int k = c16 / G;
  const bool live = k < 32 && ((pack >> k) & 1u);
  const size_t row = static_cast<size_t>(b + k) * a.num_q_heads + g * G + c16 % G;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    u32x4 w = {0u, 0u, 0u, 0u};
    if (live) w = qc[row * RC + (PERMUTED ? 4 * j + c : 4 * c + j)] ^ qsign;
    qf[c] = __builtin_bit_cast(bf16x8, w);
  }
}

// The end of a work unit: the running sum of column c16 gathered over the four
// 16-lane rows, then O / l (times vsc, the V scale of an E4M3 pool) and the
// log-sum-exp stored as the unit's partial result (split mode), or as the
// final result (single pass: W == 1) or merged across the W waves in LDS first.
// W == 1: column c16 is head g*G + c16 % G of sequence b + c16 / G, stored when
// bit c16 / G of pack is set.
template <int G, int W>
__device__ __forceinline__ void finish_unit(const DecodeArgs& a, int b, uint32_t pack, int g, int part,
                                            int wave, int lane, float m, float l, const floatx4* oacc, float vsc,
                                            float (*sm_m)[G], float (*sm_l)[G], float (*sm_acc)[G][128]) {
  constexpr int D = 128;
  const int j = lane >> 4, c16 = lane & 15;
  l = across_rows(l, OpSum());
  if constexpr (W == 1) {
    const int k = c16 / G;
    if (k >= 32 || !((pack >> k) & 1u)) return;
    const float inv = vsc / l;
    const float lse = (m + __log2f(l)) * kLn2;
    const size_t row = static_cast<size_t>(b + k) * a.num_q_heads + g * G + c16 % G;
    if (a.partition_size > 0) {
      const size_t pr = row * a.num_partitions + part;
#pragma unroll
      for (int dn = 0; dn < 8; ++dn)
        *reinterpret_cast<floatx4*>(a.part_out + pr * D + 16 * dn + 4 * j) = oacc[dn] * inv;
      if (j == 0) a.part_lse[pr] = lse;
    } else {
      uint16_t* out = static_cast<uint16_t*>(a.out);
#pragma unroll
      for (int dn = 0; dn < 8; ++dn) {
        u32x2 w;
        w[0] = pack_bf16x2(oacc[dn][0] * inv, oacc[dn][1] * inv);
        w[1] = pack_bf16x2(oacc[dn][2] * inv, oacc[dn][3] * inv);
        *reinterpret_cast<u32x2*>(out + row * D + 16 * dn + 4 * j) = w;
      }
      if (j == 0) a.lse[row] = lse;
    }
  } else {
    if (c16 < G) {
#pragma unroll
      for (int dn = 0; dn < 8; ++dn)
#pragma unroll
        for (int i = 0; i < 4; ++i) sm_acc[wave][c16][16 * dn + 4 * j + i] = oacc[dn][i] * vsc;
      if (j == 0) {
        sm_m[wave][c16] = m;
        sm_l[wave][c16] = l;
      }
    }
    __syncthreads();
    merge_and_store<true, D, G, W>(a, b, g, part, sm_m, sm_l, sm_acc);
  }
}

// Online-softmax update of one column (lane (j, c16) holds N raw scores of
// column c16, invisible ones -inf): the step max over the four 16-lane rows,
// a lazy rescale of (m, l, O) when some column's max passes m by more than
// the slack, then the probabilities exp2(s * sl2 - m) into p and their sum
// into l.  sl2 > 0 multiplies the raw scores inside the exponent's FMA and
// the max only (max(s) * c = max(s * c) for c > 0).
template <int N>
__device__ __forceinline__ void softmax_step(const float* s, float sl2, float& m, float& l, floatx4* oacc,
                                             float* p) {
  // IEEE maximum (v_maximum3_f32): compiler-visible, so its reads of the
  // matrix-core results are ordered by the compiler
  auto mx2 = [](float x, float y) { return __builtin_elementwise_maximum(x, y); };
  float t = mx2(mx2(s[0], s[1]), mx2(s[2], s[3]));
  if constexpr (N == 8) t = mx2(t, mx2(mx2(s[4], s[5]), mx2(s[6], s[7])));
  const float mx = quarter_max(t) * sl2;
  if (__builtin_amdgcn_ballot_w64(mx > m + kRescaleSlack)) {
    const float m_new = fmaxf(m, mx);
    const float alpha = m_new == kNegInf ? 1.f : fast_exp2(m - m_new);
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int dn = 0; dn < 8; ++dn) oacc[dn] *= alpha;
  }
  const float ms = m == kNegInf ? 0.f : m;   // no visible token yet (bad block ids)
#pragma unroll
  for (int i = 0; i < N; ++i) p[i] = fast_exp2(fmaf(s[i], sl2, -ms));   // masked: exp2(-inf) = 0
  float sum = (p[0] + p[1]) + (p[2] + p[3]);
  if constexpr (N == 8) sum += (p[4] + p[5]) + (p[6] + p[7]);
  l += sum;
}

// ---------------------------------------------------------------------------
// MFMA kernel: bf16, head_dim 128, block_size a multiple of 16
// ---------------------------------------------------------------------------
// W waves per workgroup: W = 1 in split-KV mode (one wave owns one partition,
// so every work unit of a launch can be resident at once and no cross-wave
// merge is needed); W = 4 for the single-pass mode (the waves take the
// sequence's blocks round-robin and meet in LDS).
//
// Per 16-token tile of KV head g:
//   S^T[16 tok x 16 col] = K[16 x 128] . Q^T   four v_mfma_f32_16x16x32_bf16;
//       lane (j, c16) reads token c16, dims 32c + 8j of the K tile as its A
//       operand, the group's query heads are the B operand columns.
//   online softmax on S^T: lane (j, c16) holds tokens 4j..4j+3 of column c16,
//       so the running max/rescale of a column stay in its own lanes; the tile
//       max needs one exchange across the four 16-lane rows.
//   O^T[128 d x 16 col] += V^T . P^T   eight v_mfma_f32_16x16x16_bf16: the
//       S^T accumulator layout is exactly the P^T B operand (4 consecutive
//       tokens of one column per lane), and V^T comes from LDS through
//       ds_read_b64_tr_b16, which hands each lane 4 consecutive tokens of one
//       dim from a row-major V tile.
// K and V tiles reach LDS by non-temporal global_load_lds_dwordx4 (no VGPRs;
// every cache byte is read once) into a ring of NS slots per wave, so NS - 1
// tiles' loads are in flight while one is computed.  Both tiles are stored
// row-major with XOR-swizzled 16-byte chunks: K chunk q of token t at q ^ t
// (conflict-free lane-linear b128 reads), V at q ^ 2*(t%8) (the eight tokens a
// transposed read touches spread over all 64 banks).
template <int G, int BS, int W, int NS>
__global__ __launch_bounds__(64 * W, W == 1 ? 3 : 1) void decode_mfma_kernel(DecodeArgs a) {
  constexpr int D = 128;
  constexpr int RC = D * 2 / 16;   // 16-byte chunks per bf16 row (16)
  constexpr int TPB = BS / 16;     // 16-token tiles per block
  typedef short short4v __attribute__((ext_vector_type(4)));

  // LDS ring, per slot and wave: K tile (4 KB) then V tile (4 KB)
  constexpr int kSlotChunks = 512;
  constexpr int kSlotBytes = kSlotChunks * 16;
  __shared__ __attribute__((aligned(16))) u32x4 ring[W][NS][kSlotChunks];
  __shared__ float sm_m[W][G];
  __shared__ float sm_l[W][G];
  __shared__ float sm_acc[W > 1 ? W : 1][G][D];

  const UnitId u = unit_id<W>(a);
  if (u.b < 0) return;
  const int g = u.g, part = u.part;
  const int wave = W > 1 ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : 0;
  const int lane = threadIdx.x & 63;
  const int j = lane >> 4, c16 = lane & 15;
  // split mode: sequences sharing this partition's blocks go in one unit
  int b = u.b;
  uint32_t pack = 1u;
  if constexpr (W == 1 && G < 16) {
    if (a.pack_shared) {
      const Pack pk = pack_of<16 / G, BS>(a, b, part, lane);
      if (pk.follower) return;
      b = __builtin_amdgcn_readfirstlane(pk.lead);
      pack = __builtin_amdgcn_readfirstlane(pk.mask);
    }
  }
  const int32_t* table = a.block_tables + static_cast<size_t>(b) * a.max_blocks_per_seq;
  const int blk_lo = a.partition_size > 0 ? part * (a.partition_size / BS) : 0;

  // First round trip: the group's queries and the first window of block ids
  // (speculative: bounded by the table row, masked below), issued before the
  // context length is needed.  The softmax scale multiplies the raw scores
  // inside the exponent's FMA and the tile max only; a negative scale is
  // folded into Q by an exact sign flip of its bf16 values, and a zero one
  // becomes the smallest normal float so that masked scores stay -inf.
  const float sl2 = fmaxf(fabsf(a.scale_log2), 1.17549435e-38f);
  const uint32_t qsign = a.scale_log2 < 0.f ? 0x80008000u : 0u;
  bf16x8 qf[4];
  load_group_queries<G, false>(a, b, pack, g, j, c16, qsign, qf);
  int ids_lo = blk_lo;   // first block of the id window; moves up under a window
  auto load_ids = [&](int w0) -> int {
    const int e = ids_lo + wave + W * (w0 + lane);
    return e < a.max_blocks_per_seq ? table[e] : -1;
  };
  int ids = load_ids(0);

  const Range r = work_range(a, b, part);
  if (r.blk_lo >= r.blk_hi) {
    if (a.partition_size == 0) store_empty<true, D, G>(a, b, g);
    return;
  }
  // a sliding window starts the span past the speculated first block
  if (r.blk_lo != ids_lo) {
    ids_lo = r.blk_lo;
    ids = load_ids(0);
  }
  {
    const int lblk = append_block(a, r, wave, W);
    if (lblk >= 0) {
      const int phys = table[lblk];
      if (phys >= 0 && phys < a.num_blocks) append_new_token<D, 2, false>(a, b, g, phys, (r.ctx - 1) % BS, lane);
    }
  }
  const int span = r.blk_hi - r.blk_lo;
  const int n_blocks = span > wave ? (span - wave + W - 1) / W : 0;

  float m = kNegInf;   // running max (log2 units) of column c16
  float l = 0.f;       // this lane's share of the running sum of column c16
  floatx4 oacc[8];     // O^T: dims 16dn + 4j + i of column c16
#pragma unroll
  for (int dn = 0; dn < 8; ++dn) oacc[dn] = floatx4{0.f, 0.f, 0.f, 0.f};

  const u32x4* kc = static_cast<const u32x4*>(a.k_cache);
  const u32x4* vc = static_cast<const u32x4*>(a.v_cache);

  // transposed-read address pieces (constant per lane): token 4j + c16/4,
  // dims 16dn + 4(c16%4) .. +3
  // (the chunk of dims 16dn + 4(c16%4) is 2dn + tr_half, stored at
  // (2dn + tr_half) ^ 2*(tok%8) = 2*(dn ^ tr_t8) + tr_half)
  const int tr_tok = 4 * j + (c16 >> 2);
  const int tr_t8 = tr_tok & 7;
  const int tr_half = (c16 & 3) >> 1;   // which 8-dim chunk of the 16-dim group
  const int tr_off = 8 * (c16 & 1);     // byte offset inside the 16-byte chunk
  // slot-0 LDS addresses of this lane's reads (other slots: + slot * kSlotBytes)
  // K row t, dim chunk q is stored at chunk q ^ t of the slot's row t; the MFMA
  // A operand of instruction c wants row c16, chunk 4c + j
  uint32_t k_addr[4];
  uint32_t v_addr[8];
#pragma unroll
  for (int c = 0; c < 4; ++c) k_addr[c] = lds_addr(&ring[wave][0][16 * c16 + ((4 * c + j) ^ c16)]);
#pragma unroll
  for (int dn = 0; dn < 8; ++dn)
    v_addr[dn] = lds_addr(&ring[wave][0][256]) + tr_tok * 256 + tr_off + tr_half * 16 + 32 * (dn ^ tr_t8);
  // Per-lane byte offsets of the tile's LDS-DMA loads from the (wave-uniform)
  // start of its rows: row 4c + j (K) / 4k + j (V) at its swizzled chunk.
  // Opaque, so that each load is a scalar base plus this 32-bit offset rather
  // than 64-bit address arithmetic per load.
  uint32_t dma_off[8];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int tok = 4 * c + j;
    dma_off[c] = static_cast<uint32_t>((tok * RC + (c16 ^ tok)) * 16);
    dma_off[4 + c] = static_cast<uint32_t>((tok * RC + (c16 ^ (2 * (tok & 7)))) * 16);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) asm volatile("" : "+v"(dma_off[i]));

  for (int w0 = 0; w0 < n_blocks; w0 += 64) {
    if (w0 > 0) ids = load_ids(w0);
    const int wn = min(64, n_blocks - w0);
    const int nt = wn * TPB;

    // Window tile n: first token position and the valid-token limit (0 when
    // the block id lies outside the pool, a precondition violation: block 0 is
    // read instead and every token masked).
    auto tile_span = [&](int n, int& pos0, int& lim, int& phys) {
      const int i = n / TPB;
      pos0 = (r.blk_lo + wave + W * (w0 + i)) * BS + (n % TPB) * 16;
      phys = __builtin_amdgcn_readlane(ids, i);
      const bool ok = phys >= 0 && phys < a.num_blocks;
      phys = ok ? phys : 0;
      lim = ok ? r.ctx : 0;
    };
    // Issue the LDS-DMA loads of window tile n into ring slot SLOT (K then V,
    // both row-major with the XOR chunk swizzle).
    auto fetch = [&](int n, auto slot_c) {
      constexpr int SLOT = decltype(slot_c)::value;
      int pos0, lim, phys;
      tile_span(n, pos0, lim, phys);
      const size_t base = ((static_cast<size_t>(phys) * a.num_kv_heads + g) * BS + (n % TPB) * 16) * RC;
      const char* kb = reinterpret_cast<const char*>(kc + base);
      const char* vb = reinterpret_cast<const char*>(vc + base);
#pragma unroll
      for (int c = 0; c < 4; ++c) global_to_lds16<PA_DECODE_AUX>(kb + dma_off[c], &ring[wave][SLOT][64 * c]);
#pragma unroll
      for (int k = 0; k < 4; ++k) global_to_lds16<PA_DECODE_AUX>(vb + dma_off[4 + k], &ring[wave][SLOT][256 + 64 * k]);
    };

    // Compute window tile n from ring slot SLOT (its loads have landed).
    auto process = [&](int n, auto slot_c) {
      constexpr int SLOT = decltype(slot_c)::value;
      constexpr int OFF = SLOT * kSlotBytes;
      int pos0, lim, phys;
      tile_span(n, pos0, lim, phys);
      u32x4 kw[4];
      u32x2 vt[8];
      // Rows past the end of the sequence may hold anything (NaN), and a zero
      // probability times NaN is still NaN: in the tile that holds the end,
      // each lane zeroes the V rows it fetched that lie past it (in LDS,
      // before the reads; LDS operations of a wave complete in order).
      if (pos0 + 16 > lim) {
        const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (pos0 + 4 * k + j >= lim) ring[wave][SLOT][256 + 64 * k + lane] = zero;
      }
      lds_read_decode_tile<OFF>(kw, vt, k_addr, v_addr);
      floatx4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c)
        st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kw[c]), qf[c], st, 0, 0, 0);
      // st[i]: raw score of token pos0 + 4j + i for column c16.  A tile wholly
      // inside the visible range (the common case) takes no mask; the others
      // set their invisible scores to -inf (a wave-uniform branch).
      const bool full = pos0 >= r.lo && pos0 + 16 <= lim;
      float s[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) s[i] = st[i];
      if (!full) {
        int d0 = pos0 + 4 * j;
        asm volatile("" : "+v"(d0));   // keeps the compares out of full tiles
#pragma unroll
        for (int i = 0; i < 4; ++i) s[i] = (d0 + i < lim && d0 + i >= r.lo) ? s[i] : kNegInf;
      }
      float p[4];
      softmax_step<4>(s, sl2, m, l, oacc, p);
      const short4v pb = __builtin_bit_cast(short4v, u32x2{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])});
#pragma unroll
      for (int dn = 0; dn < 8; ++dn)
        oacc[dn] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4v, vt[dn]), pb, oacc[dn], 0,
                                                              0, 0);
    };
    // Ring of NS slots: tile n + NS - 1's loads are issued before tile n is
    // computed, so NS - 1 tiles are in flight; the wait then lets exactly the
    // loads issued after tile n stay in flight (none after the last tile, so
    // no tile is fetched twice).  The compiler cannot count LDS-DMA
    // completions, so the waits are explicit.  Tiles go round the ring in
    // groups of NS so that every slot index is a compile-time constant.
    static_for<0, NS - 1>([&](auto k_c) {
      if (decltype(k_c)::value < nt) fetch(decltype(k_c)::value, k_c);
    });
    for (int n0 = 0; n0 < nt; n0 += NS) {
      static_for<0, NS>([&](auto k_c) {
        constexpr int K = decltype(k_c)::value;
        const int n = n0 + K;
        if (n < nt) {
          if (n + NS - 1 < nt) fetch(n + NS - 1, std::integral_constant<int, (K + NS - 1) % NS>{});
          wait_tiles_ahead<8, NS - 1>(min(NS - 1, nt - 1 - n));
          process(n, k_c);
        }
      });
    }
  }
  finish_unit<G, W>(a, b, pack, g, part, wave, lane, m, l, oacc, 1.f, sm_m, sm_l, sm_acc);
}

// ---------------------------------------------------------------------------
// MFMA kernel over E4M3 pools: head_dim 128, block_size a multiple of 16
// ---------------------------------------------------------------------------
// Work units and waves as in the bf16 kernel.  The pools hold E4M3 codes
// (128-byte rows, half the bytes), and a step takes two 16-row tiles, A and B
// (32 positions):
//   S^T of each tile: four v_mfma_f32_16x16x32_bf16.  The dot product's dims
//       run in a permuted order so that MFMA c, lane (j, c16) uses dims
//       32j + 8c .. +7 (Q is loaded in the same order): a lane's 32 K codes
//       are one contiguous run, two 16-byte reads, converted to bf16 in
//       registers.  Lane (j, c16) reads row c16 of tile A and row c16 ^ 8 of
//       tile B, so the scores a lane ends with are of rows 4j..4j+3 of A and
//       (4j..4j+3) ^ 8 of B.
//   online softmax over those eight scores per lane: one max exchange and
//       one rescale vote per step.
//   O^T += V^T . P^T: eight v_mfma_f32_16x16x32_bf16, the eight
//       probabilities of a lane its P^T operand.  V^T comes straight from the
//       codes: ds_read_b64_tr_b8 hands lane c16 of a 16-lane group byte c16 % 8
//       of the 8-byte runs that its lanes 2t + c16 / 8 address (t = 0..7), so
//       lanes 2t and 2t + 1 of group j address dims 16dn .. +15 of the row
//       behind P^T element t (A's rows for t < 4, B's after) and each lane
//       converts the 8 codes it receives to bf16.  No bf16 copy of V is made.
// Ring slot per step (8 KB, NS per wave): K_A, V_A, K_B, V_B, 16 rows x 8
// chunks each, chunk q of row r at q ^ (r / 2): the K reads of 16 lanes touch
// every bank once, and so do the transposed reads of each half-wave (16
// distinct rows, thanks to the ^ 8 for tile B).  The K scale multiplies the
// softmax scale, the V scale the output.
template <int G, int BS, int W, int NS>
__global__ __launch_bounds__(64 * W, W == 1 ? 3 : 1) void decode_fp8_kernel(DecodeArgs a) {
  constexpr int D = 128;
  constexpr int RC8 = D / 16;            // 16-byte chunks per E4M3 row (8)
  constexpr int TPB = BS / 16;           // 16-row tiles per block
  constexpr int kTile = 16 * RC8;        // chunks of one tile of one pool (128)
  constexpr int kSlotBytes = 4 * kTile * 16;
  __shared__ __attribute__((aligned(16))) u32x4 ring[W][NS][4 * kTile];
  __shared__ float sm_m[W][G];
  __shared__ float sm_l[W][G];
  __shared__ float sm_acc[W > 1 ? W : 1][G][D];

  const UnitId u = unit_id<W, true>(a);
  if (u.b < 0) return;
  const int g = u.g, b = u.b, part = u.part;
  const int wave = W > 1 ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : 0;
  const int lane = threadIdx.x & 63;
  const int j = lane >> 4, c16 = lane & 15;
  const int32_t* table = a.block_tables + static_cast<size_t>(b) * a.max_blocks_per_seq;
  const int blk_lo = a.partition_size > 0 ? part * (a.partition_size / BS) : 0;

  // scale handling as in the bf16 kernel, with the K scale folded in
  const float sl2_raw = a.scale_log2 * a.k_scale[0];
  const float sl2 = fmaxf(fabsf(sl2_raw), 1.17549435e-38f);
  const uint32_t qsign = sl2_raw < 0.f ? 0x80008000u : 0u;
  bf16x8 qf[4];
  load_group_queries<G, true>(a, b, 1u, g, j, c16, qsign, qf);
  int ids_lo = blk_lo;
  auto load_ids = [&](int w0) -> int {
    const int e = ids_lo + wave + W * (w0 + lane);
    return e < a.max_blocks_per_seq ? table[e] : -1;
  };
  int ids = load_ids(0);

  const Range r = work_range(a, b, part);
  if (r.blk_lo >= r.blk_hi) {
    if (a.partition_size == 0) store_empty<true, D, G>(a, b, g);
    return;
  }
  if (r.blk_lo != ids_lo) {
    ids_lo = r.blk_lo;
    ids = load_ids(0);
  }
  {
    const int lblk = append_block(a, r, wave, W);
    if (lblk >= 0) {
      const int phys = table[lblk];
      if (phys >= 0 && phys < a.num_blocks) append_new_token<D, 2, true>(a, b, g, phys, (r.ctx - 1) % BS, lane);
    }
  }
  const int span = r.blk_hi - r.blk_lo;
  const int n_blocks = span > wave ? (span - wave + W - 1) / W : 0;

  float m = kNegInf;
  float l = 0.f;
  floatx4 oacc[8];     // O^T: dims 16dn + 4j + i of column c16
#pragma unroll
  for (int dn = 0; dn < 8; ++dn) oacc[dn] = floatx4{0.f, 0.f, 0.f, 0.f};

  const u32x4* kc = static_cast<const u32x4*>(a.k_cache);
  const u32x4* vc = static_cast<const u32x4*>(a.v_cache);

  // slot-0 LDS addresses of this lane's reads (slot 1: + kSlotBytes).
  // K: row c16 of tile A, row c16 ^ 8 of tile B; chunks 2j and 2j + 1.
  uint32_t k_addr[4];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int rb = c16 ^ 8;
    k_addr[e] = lds_addr(&ring[wave][0][8 * c16 + ((2 * j + e) ^ (c16 >> 1))]);
    k_addr[2 + e] = lds_addr(&ring[wave][0][2 * kTile + 8 * rb + ((2 * j + e) ^ (rb >> 1))]);
  }
  // V: lane 2t + h of group j addresses the row of P^T element t (A row
  // 4j + t for t < 4, B row (4j + t - 4) ^ 8 after), dims 16dn + 8h .. +7:
  // chunk dn of the row, half h.
  uint32_t v_addr[8];
  {
    const int t = c16 >> 1, h = c16 & 1;
    const int vr = t < 4 ? 4 * j + t : (4 * j + t - 4) ^ 8;
    const int vbase = t < 4 ? kTile : 3 * kTile;
#pragma unroll
    for (int dn = 0; dn < 8; ++dn) v_addr[dn] = lds_addr(&ring[wave][0][vbase + 8 * vr + (dn ^ (vr >> 1))]) + 8 * h;
  }
  const float vsc = a.v_scale[0];
  // LDS-DMA: load i of a tile fills rows 8i + lane / 8; lane % 8 is the stored
  // chunk position, so the lane fetches source chunk (lane % 8) ^ (row / 2).
  // Byte offsets from the tile's first row, opaque as in the bf16 kernel.
  uint32_t dma_off[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = 8 * i + (lane >> 3);
    dma_off[i] = static_cast<uint32_t>((row * RC8 + ((lane & 7) ^ (row >> 1))) * 16);
    asm volatile("" : "+v"(dma_off[i]));
  }

  for (int w0 = 0; w0 < n_blocks; w0 += 64) {
    if (w0 > 0) ids = load_ids(w0);
    const int wn = min(64, n_blocks - w0);
    const int nt = wn * TPB;          // tiles of this window
    const int ns = (nt + 1) >> 1;     // steps; the last holds one tile when nt is odd

    auto tile_span = [&](int n, int& pos0, int& lim, int& phys) {
      const int i = n / TPB;
      pos0 = (r.blk_lo + wave + W * (w0 + i)) * BS + (n % TPB) * 16;
      phys = __builtin_amdgcn_readlane(ids, i);
      const bool ok = phys >= 0 && phys < a.num_blocks;
      phys = ok ? phys : 0;
      lim = ok ? r.ctx : 0;
    };
    // Issue the LDS-DMA loads of step s (tiles 2s and, if it exists, 2s + 1;
    // four loads a tile) into ring slot SLOT.
    auto fetch = [&](int s, auto slot_c) {
      constexpr int SLOT = decltype(slot_c)::value;
      static_for<0, 2>([&](auto u_c) {
        constexpr int U = decltype(u_c)::value;
        const int n = 2 * s + U;
        if (U == 0 || n < nt) {
          int pos0, lim, phys;
          tile_span(n, pos0, lim, phys);
          const size_t base = ((static_cast<size_t>(phys) * a.num_kv_heads + g) * BS + (n % TPB) * 16) * RC8;
          const char* kb = reinterpret_cast<const char*>(kc + base);
          const char* vb = reinterpret_cast<const char*>(vc + base);
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            global_to_lds16<PA_DECODE_AUX>(kb + dma_off[i], &ring[wave][SLOT][2 * U * kTile + 64 * i]);
            global_to_lds16<PA_DECODE_AUX>(vb + dma_off[i], &ring[wave][SLOT][(2 * U + 1) * kTile + 64 * i]);
          }
        }
      });
    };
    // Compute step s from ring slot SLOT (its loads have landed).
    auto process = [&](int s, auto slot_c) {
      constexpr int SLOT = decltype(slot_c)::value;
      int pa0, la, pb0 = 0, lb = 0, phys;   // a missing tile B: every row invisible
      tile_span(2 * s, pa0, la, phys);
      if (2 * s + 1 < nt) tile_span(2 * s + 1, pb0, lb, phys);
      // V rows past the end (all of a missing tile B) zeroed before the reads,
      // as in the bf16 kernel
      const u32x4 zero = {0u, 0u, 0u, 0u};
      if (pa0 + 16 > la) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
          if (pa0 + 8 * i + (lane >> 3) >= la) ring[wave][SLOT][kTile + 64 * i + lane] = zero;
      }
      if (pb0 + 16 > lb) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
          if (pb0 + 8 * i + (lane >> 3) >= lb) ring[wave][SLOT][3 * kTile + 64 * i + lane] = zero;
      }
      u32x4 k8[4];
      u32x2 v8[8];
      lds_read_fp8_step<SLOT * kSlotBytes>(k8, v8, k_addr, v_addr);
      floatx4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int e = c >> 1, w = 2 * (c & 1);
        sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, e4m3x8_to_bf16(k8[e][w], k8[e][w + 1])), qf[c], sa, 0, 0, 0);
        sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, e4m3x8_to_bf16(k8[2 + e][w], k8[2 + e][w + 1])), qf[c], sb, 0, 0, 0);
      }
      // sa[i]: raw score of position pa0 + 4j + i, sb[i]: of pb0 + (4j ^ 8) + i
      const bool full = pa0 >= r.lo && pa0 + 16 <= la && pb0 >= r.lo && pb0 + 16 <= lb;
      float sv[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv[i] = sa[i];
        sv[4 + i] = sb[i];
      }
      if (!full) {
        int da = pa0 + 4 * j, db = pb0 + ((4 * j) ^ 8);
        asm volatile("" : "+v"(da), "+v"(db));   // keeps the compares out of full steps
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sv[i] = (da + i < la && da + i >= r.lo) ? sv[i] : kNegInf;
          sv[4 + i] = (db + i < lb && db + i >= r.lo) ? sv[4 + i] : kNegInf;
        }
      }
      float p[8];
      softmax_step<8>(sv, sl2, m, l, oacc, p);
      const u32x4 pw = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                        pack_bf16x2(p[6], p[7])};
      const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
      for (int dn = 0; dn < 8; ++dn)
        oacc[dn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, e4m3x8_to_bf16(v8[dn][0], v8[dn][1])), pb, oacc[dn], 0, 0, 0);
    };
    // Ring of NS slots: step s + NS - 1's loads are issued before step s is
    // computed, and the wait lets exactly the loads of the steps after s stay
    // in flight (four per tile; only the window's last step may lack tile B).
    static_for<0, NS - 1>([&](auto k_c) {
      if (decltype(k_c)::value < ns) fetch(decltype(k_c)::value, k_c);
    });
    for (int s0 = 0; s0 < ns; s0 += NS) {
      static_for<0, NS>([&](auto k_c) {
        constexpr int K = decltype(k_c)::value;
        const int s = s0 + K;
        if (s < ns) {
          if (s + NS - 1 < ns) fetch(s + NS - 1, std::integral_constant<int, (K + NS - 1) % NS>{});
          const int after = min(NS - 1, ns - 1 - s);   // steps issued after s
          wait_vmcnt_x4<2 * (NS - 1)>(8 * after - (after > 0 && (nt & 1) && s + after == ns - 1 ? 4 : 0));
          process(s, k_c);
        }
      });
    }
  }
  finish_unit<G, W>(a, b, 1u, g, part, wave, lane, m, l, oacc, vsc, sm_m, sm_l, sm_acc);
}

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------
namespace {

// LDS ring slots per wave of the bf16 split-KV kernel (the single-pass
// kernel's four waves keep two each; the E4M3 kernel has two 32-row slots).
#ifndef PA_DECODE_SLOTS
#define PA_DECODE_SLOTS 2
#endif
#ifndef PA_DECODE_FP8_SLOTS
#define PA_DECODE_FP8_SLOTS 2
#endif

template <int G, int BS, bool KV8>
hipError_t launch_mfma_gb(const DecodeArgs& a, dim3 grid, hipStream_t s) {
  if (a.partition_size > 0) {
    // flat grid of balanced units (one per KV head and live partition, in the
    // order flat_unit defines; the kernel maps ids past the last unit to no
    // work), unit-major so the KV heads of a unit spread over the XCDs
    // A window of W keys leaves a sequence at most (W-1)/P + 2 live
    // partitions (the window's keys start anywhere inside the first one).
    DecodeArgs f = a;
    int64_t per_seq = grid.z;
    if (a.window > 0 && (a.window - 1) / a.partition_size + 2 < per_seq)
      per_seq = (a.window - 1) / a.partition_size + 2;
    int64_t nwg = static_cast<int64_t>(grid.x) * grid.y * per_seq;
    if constexpr (KV8) nwg = (nwg + 8 * grid.x - 1) / (8 * grid.x) * (8 * grid.x);   // XCD-major ids
    f.flat_units = a.num_seqs <= 64 * 16 && nwg * 64 <= 0xffffffffLL;
    // column packing needs a partition's block ids in one load per lane, and
    // leaves out the window and the append (whose rows differ per sequence)
    f.pack_shared = !KV8 && G < 16 && a.window == 0 && a.k_new == nullptr && a.partition_size / BS <= 64;
    const dim3 fg = f.flat_units ? dim3(static_cast<unsigned>(nwg)) : grid;
    if constexpr (KV8)
      hipLaunchKernelGGL((decode_fp8_kernel<G, BS, 1, PA_DECODE_FP8_SLOTS>), fg, dim3(64), 0, s, f);
    else
      hipLaunchKernelGGL((decode_mfma_kernel<G, BS, 1, PA_DECODE_SLOTS>), fg, dim3(64), 0, s, f);
  } else if constexpr (KV8) {
    hipLaunchKernelGGL((decode_fp8_kernel<G, BS, 4, 2>), grid, dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL((decode_mfma_kernel<G, BS, 4, 2>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

template <int G, bool KV8 = false>
hipError_t launch_mfma_g(const DecodeArgs& a, dim3 grid, hipStream_t s) {
  switch (a.block_size) {
    case 16: return launch_mfma_gb<G, 16, KV8>(a, grid, s);
    case 32: return launch_mfma_gb<G, 32, KV8>(a, grid, s);
    case 64: return launch_mfma_gb<G, 64, KV8>(a, grid, s);
    default: return hipErrorNotSupported;
  }
}

template <bool BF, int D>
hipError_t launch_generic_d(const DecodeArgs& a, int G, dim3 grid, hipStream_t s) {
  switch (G) {
    case 1: hipLaunchKernelGGL((decode_generic_kernel<BF, D, 1>), grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL((decode_generic_kernel<BF, D, 2>), grid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL((decode_generic_kernel<BF, D, 4>), grid, dim3(256), 0, s, a); break;
    case 8: hipLaunchKernelGGL((decode_generic_kernel<BF, D, 8>), grid, dim3(256), 0, s, a); break;
    default: return hipErrorNotSupported;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, DType dt, int head_dim, hipStream_t s) {
  const int G = a.num_q_heads / a.num_kv_heads;
  // partition slowest: every sequence's first partitions (all live) dispatch
  // before the high partitions that only long sequences have
  const dim3 grid(static_cast<unsigned>(a.num_kv_heads), static_cast<unsigned>(a.num_seqs),
                  static_cast<unsigned>(a.num_partitions));
  if (dt == DType::BF16 && head_dim == 128 && a.block_size % 16 == 0) {
    switch (G) {
      case 1: return launch_mfma_g<1>(a, grid, s);
      case 2: return launch_mfma_g<2>(a, grid, s);
      case 4: return launch_mfma_g<4>(a, grid, s);
      case 8: return launch_mfma_g<8>(a, grid, s);
      default: return hipErrorNotSupported;
    }
  }
  if (dt == DType::BF16) {
    if (head_dim == 64) return launch_generic_d<true, 64>(a, G, grid, s);
    if (head_dim == 128) return launch_generic_d<true, 128>(a, G, grid, s);
  } else {
    if (head_dim == 64) return launch_generic_d<false, 64>(a, G, grid, s);
    if (head_dim == 128) return launch_generic_d<false, 128>(a, G, grid, s);
  }
  return hipErrorNotSupported;
}

// E4M3 pools: the MFMA kernel only (bf16 queries, head_dim 128, block_size a
// multiple of 16, group 1, 2, 4 or 8).
hipError_t launch_decode_fp8(const DecodeArgs& a, int head_dim, hipStream_t s) {
  const int G = a.num_q_heads / a.num_kv_heads;
  const dim3 grid(static_cast<unsigned>(a.num_kv_heads), static_cast<unsigned>(a.num_seqs),
                  static_cast<unsigned>(a.num_partitions));
  if (head_dim != 128 || a.block_size % 16 != 0) return hipErrorNotSupported;
  switch (G) {
    case 1: return launch_mfma_g<1, true>(a, grid, s);
    case 2: return launch_mfma_g<2, true>(a, grid, s);
    case 4: return launch_mfma_g<4, true>(a, grid, s);
    case 8: return launch_mfma_g<8, true>(a, grid, s);
    default: return hipErrorNotSupported;
  }
}

// Exposed for tests of the vector-ALU kernel on shapes the MFMA kernel owns.
hipError_t launch_decode_generic(const DecodeArgs& a, DType dt, int head_dim, hipStream_t s) {
  const int G = a.num_q_heads / a.num_kv_heads;
  // partition slowest: every sequence's first partitions (all live) dispatch
  // before the high partitions that only long sequences have
  const dim3 grid(static_cast<unsigned>(a.num_kv_heads), static_cast<unsigned>(a.num_seqs),
                  static_cast<unsigned>(a.num_partitions));
  if (dt == DType::BF16) {
    if (head_dim == 64) return launch_generic_d<true, 64>(a, G, grid, s);
    if (head_dim == 128) return launch_generic_d<true, 128>(a, G, grid, s);
  } else {
    if (head_dim == 64) return launch_generic_d<false, 64>(a, G, grid, s);
    if (head_dim == 128) return launch_generic_d<false, 128>(a, G, grid, s);
  }
  return hipErrorNotSupported;
}

}  // namespace pa
