// varlen_causal_prefill: causal attention of sequences packed by cu_seqlens.
//
// The varlen call of "Llama 4 inference doubling (FlashAttention-3 +
// PagedAttention + vLLM)", section 2.4 (cumulative lengths, no padding,
// causal, returning out and lse), computed the FlashAttention way its
// section 2.4 and "PageAttention + FlashAttention golden combination",
// section 3.1 describe: tiles of Q, K and V are staged on chip, softmax and
// both matrix products are fused, and only the result goes back to HBM.
//
// prefill_mfma_kernel (bf16, head_dim 128): a workgroup owns 64 query rows of
// one (sequence, head), 16 per wave.  K/V tiles of 64 keys are double-buffered
// in LDS (K row-major, V transposed so that P.V reads 4 consecutive keys of one
// dim).  S^T = K Q^T and O^T += V^T P^T are both v_mfma_f32_16x16x32_bf16:
// the S^T accumulator layout (4 consecutive keys of one query column per lane)
// is already the B-operand layout P^T needs, so probabilities never move
// between lanes, and each lane's softmax state belongs to its own query column.
// Key tiles past the diagonal are never visited; the mask is applied on the
// diagonal tile only.  Tiles are dispatched longest-first (highest q tile
// first) so the long causal rows start early.
//
// prefill_generic_kernel (fp32 or bf16, head_dim 64/128): vector ALU, one wave
// per query row, LPT lanes per key row, online softmax per row group.
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
constexpr int kBM = 64;
constexpr int kBN = 64;
constexpr int kD = 128;
constexpr int kKP = kD + 8;    // K tile row pitch (elements): 272 B rows
constexpr int kVP = kBN + 8;   // V^T tile row pitch (elements): 144 B rows

__global__ __launch_bounds__(256, 2) void prefill_mfma_kernel(PrefillArgs a, int group) {
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][kBN * kKP];
  __shared__ __attribute__((aligned(16))) uint16_t sVt[2][kD * kVP];

  const int Hq = a.num_q_heads, Hkv = a.num_kv_heads;
  const int h = blockIdx.x % Hq;
  const int s = blockIdx.x / Hq;
  const int qt = gridDim.y - 1 - blockIdx.y;
  const SeqSpan sp = seq_span(a, s);
  const int q0 = qt * kBM;
  if (q0 >= sp.len) return;
  const int g = h / group;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int j = lane >> 4, c16 = lane & 15;
  const int my_row = q0 + wave * 16 + c16;
  const bool row_ok = my_row < sp.len;

  const u32x4* qc = static_cast<const u32x4*>(a.q);
  const u32x4* kc = static_cast<const u32x4*>(a.k);
  const u32x4* vc = static_cast<const u32x4*>(a.v);
  constexpr int RC = kD * 2 / 16;  // 16 chunks of 16 B per row

  // Q^T as the B operand: lane (j, c16) holds row my_row, dims 32c + 8j .. +7.
  bf16x8 qf[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    u32x4 w = {0u, 0u, 0u, 0u};
    if (row_ok) w = qc[(static_cast<size_t>(sp.start + my_row) * Hq + h) * RC + 4 * c + j];
    qf[c] = __builtin_bit_cast(bf16x8, w);
  }

  // Staging map: lane -> key (64 keys), wave + 4r -> 16-byte chunk (16 chunks).
  const int st_key = lane;
  u32x4 kreg[4], vreg[4];
  auto load_tile = [&](int kt) {
    const int key = kt * kBN + st_key;
    const bool ok = key < sp.len;
    const size_t rowbase = (static_cast<size_t>(sp.start + key) * Hkv + g) * RC;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int ch = wave + 4 * r;
      if (ok) {
        kreg[r] = kc[rowbase + ch];
        vreg[r] = vc[rowbase + ch];
      } else {
        kreg[r] = u32x4{0u, 0u, 0u, 0u};
        vreg[r] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int ch = wave + 4 * r;
      *reinterpret_cast<u32x4*>(&sK[buf][st_key * kKP + ch * 8]) = kreg[r];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sVt[buf][(ch * 8 + 2 * e) * kVP + st_key] = static_cast<uint16_t>(vreg[r][e] & 0xffffu);
        sVt[buf][(ch * 8 + 2 * e + 1) * kVP + st_key] = static_cast<uint16_t>(vreg[r][e] >> 16);
      }
    }
  };

  float m = kNegInf, l = 0.f;
  floatx4 oacc[8];
#pragma unroll
  for (int dn = 0; dn < 8; ++dn) oacc[dn] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int nkt = qt + 1;
  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nkt) load_tile(kt + 1);

    // S^T = K Q^T for four 16-key sub-tiles.
    floatx4 sacc[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      sacc[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const u32x4 kw = *reinterpret_cast<const u32x4*>(&sK[buf][(16 * nt + c16) * kKP + 32 * c + 8 * j]);
        sacc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kw), qf[c], sacc[nt], 0, 0, 0);
      }
    }
    // sacc[nt][i]: key kt*64 + 16nt + 4j + i, query row my_row.
    const bool diag = kt == qt;
    float mx = kNegInf;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float sv = sacc[nt][i] * a.scale_log2;
        if (diag && kt * kBN + 16 * nt + 4 * j + i > my_row) sv = kNegInf;
        sacc[nt][i] = sv;
        mx = fmaxf(mx, sv);
      }
    }
    mx = across_rows(mx, OpMax());
    const float m_new = fmaxf(m, mx);
    const float ms = m_new == kNegInf ? 0.f : m_new;
    const float alpha = fast_exp2(m - ms);
    m = m_new;
    float ps = 0.f;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = fast_exp2(sacc[nt][i] - ms);
        sacc[nt][i] = p;
        ps += p;
      }
    }
    l = l * alpha + ps;
#pragma unroll
    for (int dn = 0; dn < 8; ++dn) oacc[dn] *= alpha;

    // O^T += V^T P^T, 32 keys per MFMA: k-slot 8j+e <-> key 32kc + 4j + e (e<4),
    // 32kc + 16 + 4j + (e-4) (e>=4).
#pragma unroll
    for (int kc2 = 0; kc2 < 2; ++kc2) {
      bf16x8 pb;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pb[e] = static_cast<__bf16>(sacc[2 * kc2][e]);
        pb[e + 4] = static_cast<__bf16>(sacc[2 * kc2 + 1][e]);
      }
#pragma unroll
      for (int dn = 0; dn < 8; ++dn) {
        const uint16_t* vr = &sVt[buf][(16 * dn + c16) * kVP + 32 * kc2 + 4 * j];
        const u32x2 lo = *reinterpret_cast<const u32x2*>(vr);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(vr + 16);
        const u32x4 vw = {lo[0], lo[1], hi[0], hi[1]};
        oacc[dn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vw), pb, oacc[dn], 0, 0, 0);
      }
    }

    if (kt + 1 < nkt) store_tile(buf ^ 1);
    __syncthreads();
  }

  l = across_rows(l, OpSum());
  if (!row_ok) return;
  const float inv = 1.f / l;
  const size_t orow = static_cast<size_t>(sp.start + my_row) * Hq + h;
  uint16_t* out = static_cast<uint16_t*>(a.out);
#pragma unroll
  for (int dn = 0; dn < 8; ++dn) {
    u32x2 w;
    w[0] = pack_bf16x2(oacc[dn][0] * inv, oacc[dn][1] * inv);
    w[1] = pack_bf16x2(oacc[dn][2] * inv, oacc[dn][3] * inv);
    *reinterpret_cast<u32x2*>(out + orow * kD + 16 * dn + 4 * j) = w;
  }
  if (j == 0) a.lse[orow] = (m + __log2f(l)) * kLn2;
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
    const dim3 grid(static_cast<unsigned>(a.num_q_heads * a.num_seqs),
                    static_cast<unsigned>((a.max_seqlen + kBM - 1) / kBM));
    hipLaunchKernelGGL(prefill_mfma_kernel, grid, dim3(256), 0, s, a, group);
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
