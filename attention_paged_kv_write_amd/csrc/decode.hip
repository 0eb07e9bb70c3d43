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
// Work unit: one workgroup (4 waves) per (sequence, KV head, partition).  The
// waves of a workgroup take the partition's blocks round-robin, each keeping
// its own softmax state; the four states are merged through LDS at the end.
// The work split depends only on logical positions, never on physical block
// ids, so permuting the pool leaves every result bit-identical.
//
// Two kernels:
//  * decode_mfma_kernel (bf16, head_dim 128): QK^T of a 16-token tile against
//    the whole GQA group is one chain of four v_mfma_f32_16x16x32_bf16 (K tile
//    as the A operand, straight from HBM in MFMA layout; the group's query
//    heads as the B operand, zero-padded to 16 columns).  P.V runs on the
//    vector ALU from 16-byte V row loads, the probabilities handed over
//    through LDS.
//  * decode_generic_kernel (fp32 or bf16, head_dim 64/128): vector ALU only;
//    LPT lanes share a token row, dot products reduced with DPP.
#include "kernels.h"

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

struct Range {
  int ctx, blk_lo, blk_hi;
};

__device__ __forceinline__ Range work_range(const DecodeArgs& a, int b, int part) {
  const int cap = min(a.max_context_len, a.max_blocks_per_seq * a.block_size);
  const int ctx = clampi(a.context_lens[b], 0, cap);
  const int nblk = (ctx + a.block_size - 1) / a.block_size;
  Range r;
  r.ctx = ctx;
  if (a.partition_size > 0) {
    const int per = a.partition_size / a.block_size;
    r.blk_lo = part * per;
    r.blk_hi = min(nblk, r.blk_lo + per);
  } else {
    r.blk_lo = 0;
    r.blk_hi = nblk;
  }
  return r;
}

// Final cross-wave merge of (m, l, acc) held in LDS and the store of the result.
// sm_m/sm_l: [4][G]; sm_acc: [4][G][D].  m is in log2 units.
template <bool BF, int D, int G>
__device__ __forceinline__ void merge_and_store(const DecodeArgs& a, int b, int g, int part,
                                                const float (*sm_m)[G], const float (*sm_l)[G],
                                                const float (*sm_acc)[G][D]) {
  for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
    const int h = idx / D;
    const int e = idx - h * D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sm_m[w][h]);
    float o = 0.f, lse = kNegInf;
    if (M != kNegInf) {
      float L = 0.f, acc = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
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

  const int part = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const Range r = work_range(a, b, part);
  if (r.blk_lo >= r.blk_hi) {
    if (a.partition_size == 0) store_empty<BF, D, G>(a, b, g);
    return;
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rg = lane / LPT, dl = lane % LPT;
  const int BS = a.block_size;

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
        valid[c] = row < BS && blk * BS + row < r.ctx;
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

// ---------------------------------------------------------------------------
// MFMA kernel: bf16, head_dim 128, block_size a multiple of 16
// ---------------------------------------------------------------------------
template <int G, int BS>
__global__ __launch_bounds__(256) void decode_mfma_kernel(DecodeArgs a) {
  constexpr int D = 128;
  constexpr int RC = D * 2 / 16;   // 16-byte chunks per row (16)
  constexpr int TPB = BS / 16;     // 16-token tiles per block

  __shared__ float sm_p[4][16][G];
  __shared__ float sm_alpha[4][G];
  __shared__ float sm_m[4][G];
  __shared__ float sm_l[4][G];
  __shared__ float sm_acc[4][G][D];

  const int part = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const Range r = work_range(a, b, part);
  if (r.blk_lo >= r.blk_hi) {
    if (a.partition_size == 0) store_empty<true, D, G>(a, b, g);
    return;
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j = lane >> 4, c16 = lane & 15;

  // The group's query heads as the MFMA B operand: lane (j, c16) holds
  // q[head c16][8 dims starting at 32c + 8j] for c = 0..3; padding columns 0.
  bf16x8 qf[4];
  {
    const u32x4* qc = static_cast<const u32x4*>(a.q);
    const size_t row = static_cast<size_t>(b) * a.num_q_heads + g * G + c16;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (c16 < G) w = qc[row * RC + 4 * c + j];
      qf[c] = __builtin_bit_cast(bf16x8, w);
    }
  }

  float m = kNegInf;   // running max (log2 units) of head column c16
  float l = 0.f;       // this lane's share of the running sum
  float acc[G][8];     // P.V: rows j + 4k of each tile, dims 8*c16 .. 8*c16+7
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;

  const int span = r.blk_hi - r.blk_lo;
  const int n_tiles = (span > wave ? (span - wave + 3) >> 2 : 0) * TPB;
  const u32x4* kc = static_cast<const u32x4*>(a.k_cache);
  const u32x4* vc = static_cast<const u32x4*>(a.v_cache);
  const int32_t* table = a.block_tables + static_cast<size_t>(b) * a.max_blocks_per_seq;

  // Issue the loads of tile n: K in MFMA A layout (token c16, dims 32c + 8j),
  // V as plain rows (token j + 4k, dims 8*c16).
  auto fetch = [&](int n, u32x4* kd, u32x4* vd, int& pos0) -> bool {
    const int blk = r.blk_lo + wave + 4 * (n / TPB);
    const int tile = n % TPB;
    pos0 = blk * BS + tile * 16;
    const int phys = table[blk];
    if (phys < 0 || phys >= a.num_blocks) return false;
    const size_t base = ((static_cast<size_t>(phys) * a.num_kv_heads + g) * BS + tile * 16) * RC;
#pragma unroll
    for (int c = 0; c < 4; ++c) kd[c] = kc[base + c16 * RC + 4 * c + j];
#pragma unroll
    for (int k = 0; k < 4; ++k) vd[k] = vc[base + (j + 4 * k) * RC + c16];
    return true;
  };

  u32x4 kb[4], vb[4];
  int pos_cur = 0;
  bool ok_cur = n_tiles > 0 ? fetch(0, kb, vb, pos_cur) : false;
  for (int n = 0; n < n_tiles; ++n) {
    u32x4 kn[4], vn[4];
    int pos_next = 0;
    bool ok_next = false;
    if (n + 1 < n_tiles) ok_next = fetch(n + 1, kn, vn, pos_next);

    if (ok_cur && pos_cur < r.ctx) {
      floatx4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c)
        st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kb[c]), qf[c], st, 0, 0, 0);
      // st[i] = score of token pos_cur + 4j + i for head column c16
      float s[4];
      float mx = kNegInf;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[i] = (pos_cur + 4 * j + i < r.ctx) ? st[i] * a.scale_log2 : kNegInf;
        mx = fmaxf(mx, s[i]);
      }
      mx = across_rows(mx, OpMax());
      const float m_new = fmaxf(m, mx);
      const float ms = m_new == kNegInf ? 0.f : m_new;
      const float alpha = fast_exp2(m - ms);
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[i] = fast_exp2(s[i] - ms);
        ps += s[i];
      }
      l = l * alpha + ps;
      m = m_new;
      if (c16 < G) {
#pragma unroll
        for (int i = 0; i < 4; ++i) sm_p[wave][4 * j + i][c16] = s[i];
        if (j == 0) sm_alpha[wave][c16] = alpha;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float al = sm_alpha[wave][h];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] *= al;
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int tok = j + 4 * k;
        if (pos_cur + tok < r.ctx) {
          float vf[8];
          unpack16<true>(vb[k], vf);
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const float p = sm_p[wave][tok][h];
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(p, vf[e], acc[h][e]);
          }
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      kb[c] = kn[c];
      vb[c] = vn[c];
    }
    ok_cur = ok_next;
    pos_cur = pos_next;
  }

  // Per-wave totals: l over the four rows; acc over the four token-row groups.
  l = across_rows(l, OpSum());
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = across_rows(acc[h][e], OpSum());
  if (j == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) sm_acc[wave][h][c16 * 8 + e] = acc[h][e];
    if (c16 < G) {
      sm_m[wave][c16] = m;
      sm_l[wave][c16] = l;
    }
  }
  __syncthreads();
  merge_and_store<true, D, G>(a, b, g, part, sm_m, sm_l, sm_acc);
}

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------
namespace {

template <int G>
hipError_t launch_mfma_g(const DecodeArgs& a, dim3 grid, hipStream_t s) {
  switch (a.block_size) {
    case 16: hipLaunchKernelGGL((decode_mfma_kernel<G, 16>), grid, dim3(256), 0, s, a); break;
    case 32: hipLaunchKernelGGL((decode_mfma_kernel<G, 32>), grid, dim3(256), 0, s, a); break;
    case 64: hipLaunchKernelGGL((decode_mfma_kernel<G, 64>), grid, dim3(256), 0, s, a); break;
    default: return hipErrorNotSupported;
  }
  return hipGetLastError();
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
  const dim3 grid(static_cast<unsigned>(a.num_partitions), static_cast<unsigned>(a.num_kv_heads),
                  static_cast<unsigned>(a.num_seqs));
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

// Exposed for tests of the vector-ALU kernel on shapes the MFMA kernel owns.
hipError_t launch_decode_generic(const DecodeArgs& a, DType dt, int head_dim, hipStream_t s) {
  const int G = a.num_q_heads / a.num_kv_heads;
  const dim3 grid(static_cast<unsigned>(a.num_partitions), static_cast<unsigned>(a.num_kv_heads),
                  static_cast<unsigned>(a.num_seqs));
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
