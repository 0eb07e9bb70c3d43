// varlen_causal_prefill: causal attention of sequences packed by cu_seqlens.
//
// The varlen call of "Llama 4 inference doubling (FlashAttention-3 +
// PagedAttention + vLLM)", section 2.4 (cumulative lengths, no padding,
// causal, returning out and lse), computed the FlashAttention way its
// section 2.4 and "PageAttention + FlashAttention golden combination",
// section 3.1 describe: tiles of Q, K and V are staged on chip, softmax and
// both matrix products are fused, and only the result goes back to HBM.
//
// prefill_mfma_kernel (bf16, head_dim 128): a workgroup owns PM query rows
// (16 per wave, NR waves stacked) of NW query heads that share one KV head, so
// every K/V tile it stages serves NW * PM query rows.  K/V tiles of 64 keys are
// double-buffered in LDS by LDS-DMA (global_load_lds, no VGPR round trip), row
// major with XOR-swizzled 16-byte chunks.  S^T = K Q^T and O^T += V^T P^T are
// both v_mfma_f32_16x16x32_bf16: the S^T accumulator layout (4 consecutive
// keys of one query column per lane) is already the B-operand layout P^T
// needs, so probabilities never move between lanes and each lane's softmax
// state belongs to its own query column; V^T comes from the row-major tile by
// ds_read_b64_tr_b16.  Key tiles past the diagonal are never visited; the mask
// is applied on diagonal tiles only.
//
// Scheduling: workgroups are dealt to the 8 XCDs round-robin; the kernel maps
// its id so that one head column (KV head, head block) stays on one XCD and
// that XCD runs the q tiles of one sequence (longest first) back to back, so
// the concurrent workgroups of an XCD stream the same K/V prefix through its L2.
//
// prefill_generic_kernel (fp32 or bf16, head_dim 64/128): vector ALU, one wave
// per query row, LPT lanes per key row, online softmax per row group.
#include "kernels.h"

namespace pa {

namespace {

typedef short short4v __attribute__((ext_vector_type(4)));

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

struct SeqSpan {
  int start, len;
};

__device__ __forceinline__ SeqSpan seq_span(const PrefillArgs& a, int s) {
  const int lo = clampi(a.cu_seqlens[s], 0, a.total_tokens);
  const int hi = clampi(a.cu_seqlens[s + 1], lo, a.total_tokens);
  return SeqSpan{lo, min(hi - lo, a.max_seqlen)};
}

}  // namespace

// ---------------------------------------------------------------------------
// MFMA kernel
// ---------------------------------------------------------------------------
constexpr int kPN = 64;    // keys per K/V tile
constexpr int kD = 128;

#ifndef PA_PREFILL_NR
#define PA_PREFILL_NR 2
#endif
#ifndef PA_PREFILL_RG
#define PA_PREFILL_RG 1
#endif
#ifndef PA_PREFILL_BAND
#define PA_PREFILL_BAND 1
#endif

// Wait until this wave's LDS-DMA loads have landed.
__device__ __forceinline__ void wait_dma_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// NW waves per head-set (heads of one KV group), NR row-waves per head, RG
// 16-row groups per wave: a workgroup covers 16*RG*NR query rows of NW heads.
template <int NW, int NR, int RG>
__global__ __launch_bounds__(64 * NW * NR) void prefill_mfma_kernel(PrefillArgs a, int group, int band, int ntiles) {
  constexpr int NWAVES = NW * NR;
  constexpr int PM = 16 * RG * NR;   // query rows per workgroup
  // one K/V tile per buffer: K rows (64 x 16 chunks of 16 B) then V rows
  __shared__ __attribute__((aligned(16))) u32x4 kv0[2048];
  __shared__ __attribute__((aligned(16))) u32x4 kv1[2048];

  // Workgroup -> (head column, sequence, q tile).  Workgroups are dealt to the
  // 8 XCDs round-robin, so the XCD is the id mod 8: head column c (KV head g,
  // head block hb) lives on XCD c mod 8, and its workgroups run through bands
  // of `band` sequences, q tiles longest-first inside a band with the band's
  // sequences interleaved.  Workgroups of one band run together on one XCD
  // and stream the same K/V prefix through its L2.
  const int Hkv = a.num_kv_heads;
  const int nhb = group / NW;   // head blocks per KV group
  const int ncol = Hkv * nhb;
  const int cpx = (ncol + 7) >> 3;   // head columns per XCD
  const int id = blockIdx.x;
  const int xcd = id & 7;
  int r = id >> 3;
  const int col = (r % cpx) * 8 + xcd;
  r /= cpx;
  if (col >= ncol) return;
  const int g = col % Hkv, hb = col / Hkv;
  const int per_band = band * ntiles;
  const int bi = r / per_band, w = r % per_band;
  const int s = bi * band + w % band;
  if (s >= a.num_seqs) return;
  const int qt = ntiles - 1 - w / band;
  const SeqSpan sp = seq_span(a, s);
  const int qw0 = qt * PM;   // the workgroup's first row
  if (qw0 >= sp.len) return;
  const int wave = NWAVES > 1 ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : 0;
  const int lane = threadIdx.x & 63;
  const int j = lane >> 4, c16 = lane & 15;
  const int h = g * group + hb * NW + wave % NW;
  const int q0 = qw0 + (wave / NW) * 16 * RG;   // this wave's first row
  const int Hq = a.num_q_heads;
  constexpr int RC = kD * 2 / 16;   // 16-byte chunks per row

  const u32x4* qc = static_cast<const u32x4*>(a.q);
  const u32x4* kc = static_cast<const u32x4*>(a.k);
  const u32x4* vc = static_cast<const u32x4*>(a.v);

  // Q^T as B operands: rows q0 + 16rg + c16, dims 32c + 8j .. +7.
  bf16x8 qf[RG][4];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    const int row = q0 + 16 * rg + c16;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (row < sp.len) w = qc[(static_cast<size_t>(sp.start + row) * Hq + h) * RC + 4 * c + j];
      qf[rg][c] = __builtin_bit_cast(bf16x8, w);
    }
  }

  const int kend = min(qw0 + PM, sp.len);   // keys 0 .. kend-1 are needed by the workgroup
  const int nkt = (kend + kPN - 1) / kPN;

  // LDS-DMA of key tile kt: 2048 chunks (K then V), the NW waves take every
  // NW-th 64-chunk slice.  Position p holds row (p%1024)/16 at stored chunk
  // p%16; K chunks are XOR-swizzled by row%16 (conflict-free b128 reads of one
  // dim chunk across 8 rows), V chunks by 2*(row%8) (conflict-free transposed
  // reads).  Keys past the sequence read its last key (masked anyway).
  auto issue = [&](int kt, u32x4* buf) {
#pragma unroll 1
    for (int i = wave; i < 32; i += NWAVES) {
      const int p = 64 * i + lane;
      const bool is_v = p >= 1024;
      const int row = (p & 1023) >> 4, sc = p & 15;
      const int chunk = is_v ? (sc ^ (2 * (row & 7))) : (sc ^ (row & 15));
      const int key = min(kt * kPN + row, sp.len - 1);
      const u32x4* src = (is_v ? vc : kc) + (static_cast<size_t>(sp.start + key) * Hkv + g) * RC + chunk;
      global_to_lds16(src, &buf[64 * i]);
    }
  };

  float m[RG], l[RG];
  floatx4 oacc[RG][8];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    m[rg] = kNegInf;
    l[rg] = 0.f;
  }
#pragma unroll
  for (int rg = 0; rg < RG; ++rg)
#pragma unroll
    for (int dn = 0; dn < 8; ++dn) oacc[rg][dn] = floatx4{0.f, 0.f, 0.f, 0.f};

  // transposed-read pieces: token rows 32kc + 4j + c16/4 (+16), dims 16dn + 4(c16%4)
  const int tr_row = 4 * j + (c16 >> 2);
  const int tr_half = (c16 & 3) >> 1;
  const int tr_byte = 8 * (c16 & 1);

  auto compute = [&](int kt, const u32x4* buf) {
    // S^T = K Q^T: four 16-key sub-tiles x two 16-row groups
    floatx4 sacc[4][RG];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      // keep each sub-tile's LDS reads next to their MFMAs (register pressure)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) sacc[nt][rg] = floatx4{0.f, 0.f, 0.f, 0.f};
      const int row = 16 * nt + c16;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const u32x4 kw = buf[row * 16 + ((4 * c + j) ^ c16)];
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
          sacc[nt][rg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kw), qf[rg][c],
                                                                 sacc[nt][rg], 0, 0, 0);
      }
    }
    // sacc[nt][rg][i]: key kt*64 + 16nt + 4j + i, query row q0 + 16rg + c16
    const bool diag = kt * kPN + kPN - 1 > q0;
    short4v pb[2][RG][2];   // [kc][rg][half]: P^T B operand pieces
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
      const int qrow = q0 + 16 * rg + c16;
      float mx = kNegInf;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float sv = sacc[nt][rg][i] * a.scale_log2;
          if (diag && kt * kPN + 16 * nt + 4 * j + i > qrow) sv = kNegInf;
          sacc[nt][rg][i] = sv;
          mx = fmaxf(mx, sv);
        }
      }
      mx = across_rows(mx, OpMax());
      const float m_new = fmaxf(m[rg], mx);
      const float ms = m_new == kNegInf ? 0.f : m_new;
      const float alpha = fast_exp2(m[rg] - ms);
      m[rg] = m_new;
      float ps = 0.f;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = fast_exp2(sacc[nt][rg][i] - ms);
          ps += p;
          pb[nt >> 1][rg][nt & 1][i] = static_cast<short>(f32_to_bf16_bits(p));
        }
      }
      l[rg] = l[rg] * alpha + ps;
#pragma unroll
      for (int dn = 0; dn < 8; ++dn) oacc[rg][dn] *= alpha;
    }
    // O^T += V^T P^T, 32 keys per MFMA: k-slot 8j+e <-> key 32kc + 4j + e (e<4),
    // 32kc + 16 + 4j + (e-4) (e>=4); V^T read transposed from the row-major tile.
    const char* vbase = reinterpret_cast<const char*>(buf + 1024);
#pragma unroll
    for (int kc2 = 0; kc2 < 2; ++kc2) {
      bf16x8 pfull[RG];
#pragma unroll
      for (int rg = 0; rg < RG; ++rg)
        pfull[rg] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(pb[kc2][rg][0], pb[kc2][rg][1],
                                                                       0, 1, 2, 3, 4, 5, 6, 7));
      const int r0 = 32 * kc2 + tr_row, r1 = r0 + 16;
#pragma unroll
      for (int dn = 0; dn < 8; ++dn) {
        if ((dn & 1) == 0) __builtin_amdgcn_sched_barrier(0);
        const int ch = 2 * dn + tr_half;
        const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) short4v*)(vbase + (r0 * 16 + (ch ^ (2 * (r0 & 7)))) * 16 + tr_byte));
        const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) short4v*)(vbase + (r1 * 16 + (ch ^ (2 * (r1 & 7)))) * 16 + tr_byte));
        const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
          oacc[rg][dn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pfull[rg], oacc[rg][dn], 0, 0, 0);
      }
    }
  };

  // Double-buffered: the DMA of tile kt+1 runs while tile kt is computed.  A
  // buffer is refilled only after the barrier that follows its last reads.
  issue(0, kv0);
  for (int kt = 0; kt < nkt; kt += 2) {
    wait_dma_all();
    __syncthreads();
    if (kt + 1 < nkt) issue(kt + 1, kv1);
    compute(kt, kv0);
    if (kt + 1 >= nkt) break;
    wait_dma_all();
    __syncthreads();
    if (kt + 2 < nkt) issue(kt + 2, kv0);
    compute(kt + 1, kv1);
  }

  uint16_t* out = static_cast<uint16_t*>(a.out);
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    const float lt = across_rows(l[rg], OpSum());
    const int row = q0 + 16 * rg + c16;
    if (row < sp.len) {
      const float inv = 1.f / lt;
      const size_t orow = static_cast<size_t>(sp.start + row) * Hq + h;
#pragma unroll
      for (int dn = 0; dn < 8; ++dn) {
        u32x2 w;
        w[0] = pack_bf16x2(oacc[rg][dn][0] * inv, oacc[rg][dn][1] * inv);
        w[1] = pack_bf16x2(oacc[rg][dn][2] * inv, oacc[rg][dn][3] * inv);
        *reinterpret_cast<u32x2*>(out + orow * kD + 16 * dn + 4 * j) = w;
      }
      if (j == 0) a.lse[orow] = (m[rg] + __log2f(lt)) * kLn2;
    }
  }
}

// ---------------------------------------------------------------------------
// Vector-ALU kernel: 4 query rows per workgroup, one per wave.
// ---------------------------------------------------------------------------
template <bool BF, int D>
__global__ __launch_bounds__(256) void prefill_generic_kernel(PrefillArgs a, int group) {
  constexpr int ESZ = BF ? 2 : 4;
  constexpr int VEC = 16 / ESZ;
  constexpr int LPT = D * ESZ / 16;
  constexpr int TPW = 64 / LPT;
  constexpr int RC = D * ESZ / 16;

  const int h = blockIdx.y, s = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const SeqSpan sp = seq_span(a, s);
  const int i = blockIdx.x * 4 + wave;
  if (i >= sp.len) return;
  const int Hq = a.num_q_heads, Hkv = a.num_kv_heads;
  const int g = h / group;
  const int rg = lane / LPT, dl = lane % LPT;
  const u32x4* qc = static_cast<const u32x4*>(a.q);
  const u32x4* kc = static_cast<const u32x4*>(a.k);
  const u32x4* vc = static_cast<const u32x4*>(a.v);

  float qv[VEC];
  unpack16<BF>(qc[(static_cast<size_t>(sp.start + i) * Hq + h) * RC + dl], qv);
  float m = kNegInf, l = 0.f, acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;

  for (int k0 = 0; k0 <= i; k0 += TPW) {
    const int key = k0 + rg;
    const bool valid = key <= i;
    float kf[VEC], vf[VEC];
    if (valid) {
      const size_t rb = (static_cast<size_t>(sp.start + key) * Hkv + g) * RC + dl;
      unpack16<BF>(kc[rb], kf);
      unpack16<BF>(vc[rb], vf);
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) kf[e] = vf[e] = 0.f;
    }
    float t = 0.f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) t = fmaf(qv[e], kf[e], t);
    t = group_allreduce<LPT>(t, OpSum());
    const float sv = valid ? t * a.scale_log2 : kNegInf;
    const float m_new = fmaxf(m, sv);
    const float ms = m_new == kNegInf ? 0.f : m_new;
    const float alpha = fast_exp2(m - ms);
    const float p = fast_exp2(sv - ms);
    l = l * alpha + p;
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = fmaf(p, vf[e], acc[e] * alpha);
    m = m_new;
  }
#pragma unroll
  for (int step = LPT; step < 64; step *= 2) {
    const float mo = xchg_xor(m, step), lo = xchg_xor(l, step);
    const float M = fmaxf(m, mo);
    const float ms = M == kNegInf ? 0.f : M;
    const float f = fast_exp2(m - ms), fo = fast_exp2(mo - ms);
    l = l * f + lo * fo;
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = acc[e] * f + xchg_xor(acc[e], step) * fo;
    m = M;
  }
  if (rg != 0) return;
  const size_t orow = static_cast<size_t>(sp.start + i) * Hq + h;
  const float inv = 1.f / l;
  if constexpr (BF) {
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(acc[2 * e] * inv, acc[2 * e + 1] * inv);
    static_cast<u32x4*>(a.out)[orow * RC + dl] = w;
  } else {
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = __float_as_uint(acc[e] * inv);
    static_cast<u32x4*>(a.out)[orow * RC + dl] = w;
  }
  if (dl == 0) a.lse[orow] = (m + __log2f(l)) * kLn2;
}

hipError_t launch_prefill(const PrefillArgs& a, DType dt, int head_dim, hipStream_t s) {
  if (a.num_seqs == 0 || a.max_seqlen == 0) return hipSuccess;
  const int group = a.num_q_heads / a.num_kv_heads;
  if (dt == DType::BF16 && head_dim == kD) {
    const int nw = group >= 4 ? 4 : group;   // heads of one KV group per workgroup
    constexpr int kNR = PA_PREFILL_NR, kRG = PA_PREFILL_RG;
    constexpr int kPM = 16 * kNR * kRG;
    const int ntiles = (a.max_seqlen + kPM - 1) / kPM;
    const int ncol = a.num_kv_heads * (group / nw);
    const int band = a.num_seqs < PA_PREFILL_BAND ? a.num_seqs : PA_PREFILL_BAND;
    const int64_t nb = (a.num_seqs + band - 1) / band;
    const int64_t n = 8LL * ((ncol + 7) / 8) * nb * band * ntiles;
    if (n * 64 * nw * kNR > 0xffffffffLL) return hipErrorInvalidValue;   // total threads of a launch
    const dim3 grid(static_cast<unsigned>(n));
    switch (nw) {
      case 4: hipLaunchKernelGGL((prefill_mfma_kernel<4, kNR, kRG>), grid, dim3(256 * kNR), 0, s, a, group, band, ntiles); break;
      case 2: hipLaunchKernelGGL((prefill_mfma_kernel<2, kNR, kRG>), grid, dim3(128 * kNR), 0, s, a, group, band, ntiles); break;
      default: hipLaunchKernelGGL((prefill_mfma_kernel<1, kNR, kRG>), grid, dim3(64 * kNR), 0, s, a, group, band, ntiles); break;
    }
    return hipGetLastError();
  }
  return launch_prefill_generic(a, dt, head_dim, s);
}

hipError_t launch_prefill_generic(const PrefillArgs& a, DType dt, int head_dim, hipStream_t s) {
  if (a.num_seqs == 0 || a.max_seqlen == 0) return hipSuccess;
  const int group = a.num_q_heads / a.num_kv_heads;
  const dim3 grid(static_cast<unsigned>((a.max_seqlen + 3) / 4), static_cast<unsigned>(a.num_q_heads),
                  static_cast<unsigned>(a.num_seqs));
  if (dt == DType::BF16) {
    if (head_dim == 64) hipLaunchKernelGGL((prefill_generic_kernel<true, 64>), grid, dim3(256), 0, s, a, group);
    else if (head_dim == 128) hipLaunchKernelGGL((prefill_generic_kernel<true, 128>), grid, dim3(256), 0, s, a, group);
    else return hipErrorNotSupported;
  } else {
    if (head_dim == 64) hipLaunchKernelGGL((prefill_generic_kernel<false, 64>), grid, dim3(256), 0, s, a, group);
    else if (head_dim == 128) hipLaunchKernelGGL((prefill_generic_kernel<false, 128>), grid, dim3(256), 0, s, a, group);
    else return hipErrorNotSupported;
  }
  return hipGetLastError();
}

}  // namespace pa
