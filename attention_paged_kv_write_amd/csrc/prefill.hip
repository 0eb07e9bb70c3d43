// varlen_causal_prefill: causal attention of sequences packed by cu_seqlens.
//
// The varlen call of "Llama 4 inference doubling (FlashAttention-3 +
// PagedAttention + vLLM)", section 2.4 (cumulative lengths, no padding,
// causal, returning out and lse), computed the FlashAttention way its
// section 2.4 and "PageAttention + FlashAttention golden combination",
// section 3.1 describe: tiles of Q, K and V are staged on chip, softmax and
// both matrix products are fused, and only the result goes back to HBM.
//
// prefill_mfma_kernel (bf16, head_dim 128): a workgroup of four waves owns PM
// query rows (32 per wave, NR = 4 / NW waves stacked) of NW query heads that
// share one KV head, so every K/V tile it stages serves NW * PM query rows.  K/V tiles of 64 keys are
// double-buffered in LDS by LDS-DMA (global_load_lds, no VGPR round trip), row
// major with XOR-swizzled 16-byte chunks.  S^T = K Q^T and O^T += V^T P^T are
// both v_mfma_f32_16x16x32_bf16: the S^T accumulator layout (4 consecutive
// keys of one query column per lane) is already the B-operand layout P^T
// needs, so probabilities never move between lanes and each lane's softmax
// state belongs to its own query column; V^T comes from the row-major tile by
// ds_read_b64_tr_b16.  Key tiles past the diagonal are never visited; the mask
// is applied on diagonal tiles only.  Q comes in and O goes out through LDS as
// well, so that every global access moves whole 256-byte rows (a row per 16
// lanes) instead of 32-64-byte pieces of 16 rows.
//
// Scheduling: workgroups are dealt to the 8 XCDs round-robin; the kernel maps
// its id so that one head column (KV head, head block) stays on one XCD (or,
// with fewer than 8 columns, on the XCDs that share it) and that XCD runs the
// q tiles of one sequence (longest first) back to back, so the concurrent
// workgroups of an XCD stream the same K/V prefix through its L2.
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

// Keys of sequence s: positions 0 .. ctx-1, the first query row at position
// pos0 (so row r sees keys 0 .. pos0 + r).  Varlen: the sequence's own rows,
// pos0 = 0.  Paged: its cached positions (capped at what the table and
// max_context_len allow), the chunk being the last len of them; ctx < len is
// a precondition violation, reported as ctx = 0 (the rows are skipped).
struct KeySpan {
  int ctx, pos0;
};

template <bool PAGED>
__device__ __forceinline__ KeySpan key_span(const PrefillArgs& a, int s, int len) {
  if constexpr (!PAGED) {
    return KeySpan{len, 0};
  } else {
    const int cap = min(a.max_context_len, a.max_blocks_per_seq * a.block_size);
    const int ctx = clampi(a.context_lens[s], 0, cap);
    if (ctx < len) return KeySpan{0, 0};
    return KeySpan{ctx, ctx - len};
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// MFMA kernel
// ---------------------------------------------------------------------------
constexpr int kPN = 64;    // keys per K/V tile
constexpr int kD = 128;

// Wait until this wave's LDS-DMA loads have landed.
__device__ __forceinline__ void wait_dma_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// Wait until this wave's LDS operations have completed.
__device__ __forceinline__ void wait_lds_all() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Max / sum over lanes l, l^16, l^32, l^48 (the four key quarters of a query
// column) with VALU lane swaps.
template <class Op>
__device__ __forceinline__ float quarter_reduce(float x, Op op) {
  const auto p16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = op(__uint_as_float(p16[0]), __uint_as_float(p16[1]));
  const auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return op(__uint_as_float(p32[0]), __uint_as_float(p32[1]));
}

// Four waves per workgroup: NW query heads of one KV group times 4/NW row
// blocks; each wave owns 32 query rows (two 16-row groups) of one head, so a
// K/V fragment read from LDS feeds two MFMAs.
template <int NW, bool PAGED>
__global__ __launch_bounds__(256, 2) void prefill_mfma_kernel(PrefillArgs a, int group, int ntiles, int ksub) {
  constexpr int NR = 4 / NW;
  constexpr int PM = 32 * NR;   // query rows per workgroup
  constexpr int RG = 2;         // 16-row groups per wave
  // two K/V tiles: per tile K rows (64 x 16 chunks of 16 B) then V rows
  __shared__ __attribute__((aligned(16))) u32x4 kvbuf[2 * 2048];

  // Workgroup -> (head column, sequence, q tile).  Workgroups are dealt to
  // the 8 XCDs round-robin (the XCD is the id mod 8), and the column is the
  // id mod ncol, so with ncol a multiple of 8 head column c (KV head g, head
  // block hb) lives on XCD c mod 8.  With ncol a divisor of 8, 8 / ncol XCDs
  // share a column: when the launcher expects that to stay even (ksub = 8 /
  // ncol) XCD col + k * ncol takes the sequences s = k mod ksub whole;
  // otherwise (ksub = 1) a column's consecutive items alternate over its
  // XCDs, each taking every (8 / ncol)-th q tile of every sequence, so that
  // one long sequence or a few uneven ones still spread evenly.  Either way
  // an XCD's workgroups run sequence by sequence, q tiles longest-first
  // within a sequence, its concurrent workgroups stream the same K/V prefix
  // through its L2, and every XCD has work.
  const int Hkv = a.num_kv_heads;
  const int nhb = group / NW;   // head blocks per KV group
  const int ncol = Hkv * nhb;
  const int id = blockIdx.x;
  const int col = id % ncol;
  const int g = col % Hkv, hb = col / Hkv;
  int s, w;
  if (ksub > 1) {
    const int t = id / ncol;
    const int u = t / ksub;
    w = u % ntiles;
    s = (u / ntiles) * ksub + t % ksub;
  } else {
    const int r = id / ncol;
    s = r / ntiles;
    w = r % ntiles;
  }
  if (s >= a.num_seqs) return;
  const SeqSpan sp = seq_span(a, s);
  const int qt = (sp.len + PM - 1) / PM - 1 - w;
  if (qt < 0) return;
  const int qw0 = qt * PM;   // the workgroup's first row
  const KeySpan ks = key_span<PAGED>(a, s, sp.len);
  if (ks.ctx == 0) return;
  const int win = a.window;   // sliding window in keys, 0 = none
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int j = lane >> 4, c16 = lane & 15;
  const int h = g * group + hb * NW + wave % NW;
  const int q0 = qw0 + (wave / NW) * 32;   // this wave's first row
  const int Hq = a.num_q_heads;
  constexpr int RC = kD * 2 / 16;   // 16-byte chunks per row

  const u32x4* qc = static_cast<const u32x4*>(a.q);
  const u32x4* kc = static_cast<const u32x4*>(a.k);
  const u32x4* vc = static_cast<const u32x4*>(a.v);

  // Scores are reduced unscaled; a negative scale is folded into Q (exact
  // sign flip of the bf16 values) so the max of raw scores is the max of
  // scaled ones.
  // (a zero scale becomes the smallest normal float: every score times it
  // still rounds to nothing in the exponent, and masked keys stay -inf
  // instead of -inf * 0 = NaN)
  const float sl2 = fmaxf(fabsf(a.scale_log2), 1.17549435e-38f);
  const uint32_t qsign = a.scale_log2 < 0.f ? 0x80008000u : 0u;

  bf16x8 qf[RG][4];   // Q^T B operands, loaded below (after the first tile is requested)
  const int kend = min(ks.pos0 + qw0 + PM, ks.ctx);   // keys 0 .. kend-1 are needed by the workgroup
  const int nkt = (kend + kPN - 1) / kPN;
  // Under a window no row of the workgroup sees a key before kmin (its first
  // row's window start): tile slots below it load key kmin instead (masked),
  // so blocks wholly before the window are never touched and may be freed.
  const int kmin = win > 0 ? max(0, ks.pos0 + qw0 - win + 1) : 0;
  const unsigned wlim = win > 0 ? static_cast<unsigned>(win) : 0x7fffffffu;   // visible: 0 <= pos - key < wlim

  // LDS-DMA of key tile kt: 2048 chunks (K then V); wave w issues slices
  // w, w+4, ..., each 64 lanes x 16 B.  Slice i holds rows 4(i%16) + lane/16 at
  // stored chunk lane%16; K chunks are XOR-swizzled by row%16 (conflict-free
  // b128 reads of one dim chunk across rows), V chunks by 2*(row%8)
  // (conflict-free transposed reads).  Keys past the sequence read its last
  // key (masked anyway).
  const int drow = 4 * wave + j;   // row of slice `wave`; later slices add 16
  const int kchunk = c16 ^ (drow & 15);
  const int vchunk = c16 ^ (2 * (drow & 7));
  // Paged: the physical blocks of this lane's four rows of a tile, loaded one
  // tile ahead of its DMA (ids_next) so the table read never delays it.
  const int32_t* table = PAGED ? a.block_tables + static_cast<size_t>(s) * a.max_blocks_per_seq : nullptr;
  const int lbs = PAGED ? __builtin_ctz(a.block_size) : 0;
  int ids_cur[4] = {0, 0, 0, 0}, ids_next[4] = {0, 0, 0, 0};
  // A whole tile (no clamped key) with blocks of at least 16 keys: each DMA
  // slice of 16 rows lies in one block, so its table entry is wave-uniform
  // (a scalar load) and the lane's part of the address is a constant 32-bit
  // offset.  Other tiles take per-lane table entries.
  auto whole_tile = [&](int kt) { return kt * kPN >= kmin && kt * kPN + kPN <= ks.ctx; };
  const bool uniform_blocks = PAGED && a.block_size >= 16;
  auto load_ids = [&](int kt, int (&ids)[4]) {
    if constexpr (PAGED) {
      if (uniform_blocks && whole_tile(kt)) {
#pragma unroll
        for (int mm = 0; mm < 4; ++mm) ids[mm] = table[(kt * kPN + 16 * mm) >> lbs];
      } else {
#pragma unroll
        for (int mm = 0; mm < 4; ++mm) ids[mm] = table[min(max(kt * kPN + drow + 16 * mm, kmin), ks.ctx - 1) >> lbs];
      }
    }
  };
  auto issue = [&](int kt, u32x4* buf) {
    if constexpr (PAGED) {
      if (uniform_blocks && whole_tile(kt)) {
        uint32_t lo0 = static_cast<uint32_t>(drow * RC * 16);
        asm volatile("" : "+v"(lo0));
#pragma unroll
        for (int ii = 0; ii < 8; ++ii) {
          const int mm = ii & 3;
          int phys = __builtin_amdgcn_readfirstlane(ids_cur[mm]);
          phys = (phys >= 0 && phys < a.num_blocks) ? phys : 0;   // bad ids read block 0 (result unspecified)
          const size_t base = ((static_cast<size_t>(phys) * Hkv + g) * a.block_size +
                               ((kt * kPN + 16 * mm) & (a.block_size - 1))) * RC;
          const char* src = reinterpret_cast<const char*>((ii < 4 ? kc : vc) + base);
          global_to_lds16(src + lo0 + static_cast<uint32_t>((ii < 4 ? kchunk : vchunk) * 16), &buf[64 * (wave + 4 * ii)]);
        }
        return;
      }
    }
    if constexpr (!PAGED) {
      if (kt * kPN >= kmin && kt * kPN + kPN <= ks.ctx) {
        // The whole tile lies inside the sequence: one wave-uniform base and
        // a 32-bit offset per lane (scalar base + vector offset addressing,
        // no 64-bit address arithmetic per load).  The lane part is opaque so
        // that it is not hoisted out of the key loop as 64-bit addresses.
        const size_t t0 = (static_cast<size_t>(sp.start + kt * kPN) * Hkv + g) * RC;
        const char* kb = reinterpret_cast<const char*>(kc + t0);
        const char* vb = reinterpret_cast<const char*>(vc + t0);
        uint32_t lo0 = static_cast<uint32_t>(drow * Hkv * RC * 16);
        asm volatile("" : "+v"(lo0));
#pragma unroll
        for (int ii = 0; ii < 8; ++ii) {
          const uint32_t off = lo0 + static_cast<uint32_t>((16 * (ii & 3) * Hkv * RC + (ii < 4 ? kchunk : vchunk)) * 16);
          global_to_lds16((ii < 4 ? kb : vb) + off, &buf[64 * (wave + 4 * ii)]);
        }
        return;
      }
    }
#pragma unroll
    for (int ii = 0; ii < 8; ++ii) {
      const int row = drow + 16 * (ii & 3);
      const int key = min(max(kt * kPN + row, kmin), ks.ctx - 1);
      size_t rowoff;
      if constexpr (PAGED) {
        int phys = ids_cur[ii & 3];
        phys = (phys >= 0 && phys < a.num_blocks) ? phys : 0;   // bad ids read block 0 (result unspecified)
        rowoff = ((static_cast<size_t>(phys) * Hkv + g) * a.block_size + (key & (a.block_size - 1))) * RC;
      } else {
        rowoff = (static_cast<size_t>(sp.start + key) * Hkv + g) * RC;
      }
      const u32x4* src = ii < 4 ? kc + rowoff + kchunk : vc + rowoff + vchunk;
      global_to_lds16(src, &buf[64 * (wave + 4 * ii)]);
    }
  };

  float m[RG], l[RG];
  floatx4 oacc[RG][8];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    m[rg] = kNegInf;
    l[rg] = 0.f;
#pragma unroll
    for (int dn = 0; dn < 8; ++dn) oacc[rg][dn] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  // LDS byte offsets into kvbuf (tile 0; tile 1 adds 32 KB).
  const char* lds = reinterpret_cast<const char*>(kvbuf);
  uint32_t koff[4];   // K chunk (4c + j) ^ c16 of row c16 (+16 rows per nt)
#pragma unroll
  for (int c = 0; c < 4; ++c) koff[c] = c16 * 256 + 16 * ((4 * c + j) ^ c16);
  // transposed V reads: token row 4j + c16/4 (+32 per key chunk, +16 for the
  // second half), dims 16dn + 4(c16%4), i.e. chunk 2dn + (c16%4)/2 stored at
  // XOR 2*(row%8)
  const int tr_row = 4 * j + (c16 >> 2);
  uint32_t voff[8];
#pragma unroll
  for (int dn = 0; dn < 8; ++dn)
    voff[dn] = 16384 + tr_row * 256 + 32 * (dn ^ (tr_row & 7)) + 16 * ((c16 & 3) >> 1) + 8 * (c16 & 1);

  auto tile = [&](int kt, bool masked) {
    const uint32_t boff = (kt & 1) * 32768;
    // S^T = K Q^T: sacc[nt][rg][i] = key kt*64 + 16nt + 4j + i, row q0 + 16rg + c16
    floatx4 sacc[4][RG];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) sacc[nt][rg] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const u32x4 kw = *reinterpret_cast<const u32x4*>(lds + koff[c] + boff + 4096 * nt);
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
          sacc[nt][rg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kw), qf[rg][c],
                                                                 sacc[nt][rg], 0, 0, 0);
      }
    }
    bf16x8 pf[2][RG];   // P^T B operands: [key chunk of 32][rg]
    // Raw scores: the scale (positive here) is applied after the max,
    // max(s) * scale == max(s * scale) exactly, and inside the exponent's FMA.
    // The maxima are IEEE maximum (v_maximum3_f32), which the compiler builds
    // without NaN-quieting copies and whose reads of the matrix-core results it
    // orders itself.
    float sv[RG][4][4], lmx[RG];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
      // The row's position (among the keys) minus this lane's first key of the
      // tile, kt*64 + 4j: key kt*64 + 4j + 16nt + i is visible iff
      // 0 <= d - (16nt + i) < wlim, one unsigned compare per element.
      const int d = ks.pos0 + q0 + 16 * rg + c16 - kt * kPN - 4 * j;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[rg][nt][i] = sacc[nt][rg][i];
      if (masked) {
        // (opaque, so that the compares are not hoisted into unmasked tiles)
        int dm = d;
        asm volatile("" : "+v"(dm));
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (static_cast<unsigned>(dm - (16 * nt + i)) >= wlim) sv[rg][nt][i] = kNegInf;
      }
      auto mx2 = [](float x, float y) { return __builtin_elementwise_maximum(x, y); };
      const float(&v)[4][4] = sv[rg];
      lmx[rg] = mx2(mx2(mx2(mx2(v[0][0], v[0][1]), mx2(v[0][2], v[0][3])),
                        mx2(mx2(v[1][0], v[1][1]), mx2(v[1][2], v[1][3]))),
                    mx2(mx2(mx2(v[2][0], v[2][1]), mx2(v[2][2], v[2][3])),
                        mx2(mx2(v[3][0], v[3][1]), mx2(v[3][2], v[3][3]))));
    }
    // Lazy rescale: a row moves its maximum only when its tile max has grown
    // past the slack.  Some row's max exceeds its m + slack exactly when some
    // lane's own max does (the four lanes of a row hold the same m), so one
    // ballot of lane maxima over both row groups decides, and the row maxima
    // (across the four key quarters) are formed only on that rare path.  A row
    // with no visible key in a masked tile has max -inf and keeps its m, which
    // stays -inf until the row's first visible key (possible only under a
    // sliding window).
    if (__builtin_amdgcn_ballot_w64((lmx[0] * sl2 > m[0] + kRescaleSlack) |
                                   (lmx[1] * sl2 > m[1] + kRescaleSlack))) {
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) {
        const float mx = quarter_max(lmx[rg]) * sl2;
        if (__builtin_amdgcn_ballot_w64(mx > m[rg] + kRescaleSlack)) {
          const float m_new = fmaxf(m[rg], mx);
          const float alpha = m_new == kNegInf ? 1.f : fast_exp2(m[rg] - m_new);
          m[rg] = m_new;
          l[rg] *= alpha;
#pragma unroll
          for (int dn = 0; dn < 8; ++dn) oacc[rg][dn] *= alpha;
        }
      }
    }
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
      const float ms = m[rg] == kNegInf ? 0.f : m[rg];
      uint32_t pw[4][2];
      float ps[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        float pv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pv[i] = fast_exp2(fmaf(sv[rg][nt][i], sl2, -ms));   // masked: exp2(-inf) = 0
        ps[nt] = (pv[0] + pv[1]) + (pv[2] + pv[3]);
        pw[nt][0] = pack_bf16x2(pv[0], pv[1]);
        pw[nt][1] = pack_bf16x2(pv[2], pv[3]);
      }
#pragma unroll
      for (int kc2 = 0; kc2 < 2; ++kc2)
        pf[kc2][rg] = __builtin_bit_cast(bf16x8, u32x4{pw[2 * kc2][0], pw[2 * kc2][1], pw[2 * kc2 + 1][0],
                                                       pw[2 * kc2 + 1][1]});
      l[rg] += (ps[0] + ps[1]) + (ps[2] + ps[3]);   // this lane's quarter of the row sum, fp32
    }
    // O^T += V^T P^T, 32 keys per MFMA: k-slot 8j+e <-> key 32kc + 4j + e (e<4),
    // 32kc + 16 + 4j + (e-4) (e>=4); V^T read transposed from the row-major tile.
#pragma unroll
    for (int kc2 = 0; kc2 < 2; ++kc2) {
#pragma unroll
      for (int dn = 0; dn < 8; ++dn) {
        typedef __attribute__((address_space(3))) short4v* lds_s4;
        const char* va0 = lds + voff[dn] + boff + 8192 * kc2;
        const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4)(va0));
        const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4)(va0 + 4096));
        const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
          oacc[rg][dn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pf[kc2][rg], oacc[rg][dn], 0, 0, 0);
      }
    }
  };

  // Double-buffered: the DMA of tile kt+1 runs while tile kt is computed.  A
  // buffer is refilled only after the barrier that follows its last reads.
  // The wave's rows sit at key positions P0 .. P0 + 31 (P0 = pos0 + q0): key
  // tiles below (P0 + 1) / 64 are wholly visible, those up to the last live
  // row's position need the causal mask (one tile when pos0 = 0, since q0 is
  // a multiple of 32; at most two otherwise), later ones are skipped (every
  // wave still joins each barrier).
  // A sliding window of `win` keys also hides keys <= position - win: tiles
  // before the first row's window are skipped, tiles that reach into the last
  // row's window start are masked.  The workgroup starts at its first wave's
  // first needed tile.
  const bool wave_live = sp.len > q0;   // else every row of the wave is padding
  const int p_first = ks.pos0 + q0, p_last = ks.pos0 + min(q0 + 31, sp.len - 1);
  const int kt_first = win > 0 ? max(0, p_first - win + 1) >> 6 : 0;
  const int kt_wfull = win > 0 ? (max(0, p_last - win + 1) + kPN - 1) >> 6 : 0;
  const int kt_cfull = wave_live ? (p_first + 1) >> 6 : 0;   // tiles below are causally full
  const int kt_last = wave_live ? p_last >> 6 : -1;
  const int kt0 = kmin >> 6;
  // Q rows of this wave go through LDS: the slot tile kt0 + 1 will use is free
  // until after the first barrier, and a wave's 32 rows (8 KB) take a quarter
  // of it.  Each DMA moves four whole 256-byte rows (16 lanes per row), and
  // lane l of DMA i fetches chunk (l mod 16) ^ (row mod 16) so that the MFMA
  // operand reads below are conflict-free.  Rows past the sequence load its
  // last row and are zeroed afterwards.
  {
    u32x4* qbuf = kvbuf + ((kt0 + 1) & 1) * 2048 + wave * 512;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int rl = 4 * i + (lane >> 4);
      const int row = min(q0 + rl, sp.len - 1);
      global_to_lds16(qc + (static_cast<size_t>(sp.start + row) * Hq + h) * RC + ((lane & 15) ^ (rl & 15)),
                      &qbuf[64 * i]);
    }
  }
  load_ids(kt0, ids_cur);
  issue(kt0, kvbuf + (kt0 & 1) * 2048);
  if (kt0 + 1 < nkt) load_ids(kt0 + 1, ids_next);
  wait_dma_all();
  __syncthreads();

  // Q^T as B operands: rows q0 + 16rg + c16, dims 32c + 8j .. +7.
  {
    const u32x4* qbuf = kvbuf + ((kt0 + 1) & 1) * 2048 + wave * 512;
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
      const bool live = q0 + 16 * rg + c16 < sp.len;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const u32x4 zero = {0u, 0u, 0u, 0u};
        const u32x4 w = qbuf[(16 * rg + c16) * 16 + ((4 * c + j) ^ c16)];
        qf[rg][c] = __builtin_bit_cast(bf16x8, live ? (w ^ qsign) : zero);
      }
    }
  }
  wait_lds_all();
  __syncthreads();   // every wave holds its Q: the slot may be refilled

  for (int kt = kt0; kt < nkt; ++kt) {
    if (kt + 1 < nkt) {
#pragma unroll
      for (int mm = 0; mm < 4; ++mm) ids_cur[mm] = ids_next[mm];
      issue(kt + 1, kvbuf + ((kt + 1) & 1) * 2048);
      if (kt + 2 < nkt) load_ids(kt + 2, ids_next);
    }
    // (kt_wfull >= kt_first and kt_cfull <= kt_last + 1, so the unmasked range
    // lies inside the visible one; this form of the test also keeps the loop
    // within the register budget, which a skip-first form does not)
    // One tile body for both kinds (the mask is a wave-uniform branch over the
    // scores only): two inlined bodies made the compiler copy all of O between
    // registers at every iteration.
    if (kt >= kt_first && kt <= kt_last) tile(kt, !(kt >= kt_wfull && kt < kt_cfull));
    wait_dma_all();
    __syncthreads();
  }

  // O goes out through LDS as well (every wave is past its last tile read): the
  // wave writes its 32 normalised rows into its own 8 KB (16-byte chunk k of
  // row r at k ^ (r mod 16)), then stores four whole rows per instruction.
  // (The lane index is made opaque here so that the compiler builds these
  // addresses after the loop instead of holding them in registers through it.)
  int el = lane;
  asm volatile("" : "+v"(el));
  const int ej = el >> 4, e16 = el & 15;
  u32x4* obuf = kvbuf + wave * 512;
  char* obytes = reinterpret_cast<char*>(obuf);
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    const float lt = quarter_reduce(l[rg], OpSum());
    const int rl = 16 * rg + e16;
    const float inv = 1.f / lt;
#pragma unroll
    for (int dn = 0; dn < 8; ++dn) {
      u32x2 wo;
      wo[0] = pack_bf16x2(oacc[rg][dn][0] * inv, oacc[rg][dn][1] * inv);
      wo[1] = pack_bf16x2(oacc[rg][dn][2] * inv, oacc[rg][dn][3] * inv);
      *reinterpret_cast<u32x2*>(obytes + rl * 256 + 16 * ((2 * dn + (ej >> 1)) ^ e16) + 8 * (ej & 1)) = wo;
    }
    const int row = q0 + rl;
    if (ej == 0 && row < sp.len)
      a.lse[static_cast<size_t>(sp.start + row) * Hq + h] = (m[rg] + __log2f(lt)) * kLn2;
  }
  u32x4* oc = static_cast<u32x4*>(a.out);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int rl = 4 * i + ej;
    const u32x4 w = obuf[rl * 16 + (e16 ^ (rl & 15))];
    if (q0 + rl < sp.len) oc[(static_cast<size_t>(sp.start + q0 + rl) * Hq + h) * RC + e16] = w;
  }
}

// ---------------------------------------------------------------------------
// Vector-ALU kernel: 4 query rows per workgroup, one per wave.
// ---------------------------------------------------------------------------
template <bool BF, int D, bool PAGED>
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
  const KeySpan ks = key_span<PAGED>(a, s, sp.len);
  if (ks.ctx == 0) return;
  const int last = ks.pos0 + i;   // the row sees keys first .. last
  const int first = a.window > 0 ? max(0, last - a.window + 1) : 0;
  const int32_t* table = PAGED ? a.block_tables + static_cast<size_t>(s) * a.max_blocks_per_seq : nullptr;
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

  for (int k0 = first; k0 <= last; k0 += TPW) {
    const int key = k0 + rg;
    const bool valid = key <= last;
    float kf[VEC], vf[VEC];
    if (valid) {
      size_t rb;
      if constexpr (PAGED) {
        int phys = table[key / a.block_size];
        phys = (phys >= 0 && phys < a.num_blocks) ? phys : 0;
        rb = ((static_cast<size_t>(phys) * Hkv + g) * a.block_size + key % a.block_size) * RC + dl;
      } else {
        rb = (static_cast<size_t>(sp.start + key) * Hkv + g) * RC + dl;
      }
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

namespace {

template <bool PAGED>
hipError_t launch_mfma(const PrefillArgs& a, int group, hipStream_t s) {
  const int nw = group >= 4 ? 4 : group;   // heads of one KV group per workgroup
  const int pm = 32 * (4 / nw);            // query rows per workgroup
  const int ntiles = (a.max_seqlen + pm - 1) / pm;
  const int ncol = a.num_kv_heads * (group / nw);
  // XCDs sharing a column (ncol a divisor of 8) take whole sequences when
  // that should keep them even: at least one sequence each, and either
  // lengths close to equal (mean at least 0.8 of the maximum) or sixteen
  // sequences or more each.  Dealt against interleaved, 2 columns, same box:
  // 64 x 512 tokens 498-500 against 408 TFLOP/s, 16 x 2,048 757-798 against
  // 651-674, 128 sequences of 64-1,024 tokens 508-510 against 402-422; the
  // 16 uneven sequences of the Llama-3-8B varlen mix (mean 0.6 of the
  // maximum), where dealing leaves one XCD pair 1.38x the mean work, 479-486
  // against 523-530; one 8,192-token sequence 261 against 670.
  const int share = (ncol < 8 && 8 % ncol == 0) ? 8 / ncol : 1;
  const int64_t S = a.num_seqs;
  const bool even = 5LL * a.total_tokens >= 4LL * S * a.max_seqlen || S >= 16LL * share;
  const int ksub = (share > 1 && S >= share && even) ? share : 1;
  const int64_t n = static_cast<int64_t>(ncol) * ksub * ((a.num_seqs + ksub - 1) / ksub) * ntiles;
  if (n * 256 > 0xffffffffLL) return hipErrorInvalidValue;   // total threads of a launch
  const dim3 grid(static_cast<unsigned>(n));
  switch (nw) {
    case 4: hipLaunchKernelGGL((prefill_mfma_kernel<4, PAGED>), grid, dim3(256), 0, s, a, group, ntiles, ksub); break;
    case 2: hipLaunchKernelGGL((prefill_mfma_kernel<2, PAGED>), grid, dim3(256), 0, s, a, group, ntiles, ksub); break;
    default: hipLaunchKernelGGL((prefill_mfma_kernel<1, PAGED>), grid, dim3(256), 0, s, a, group, ntiles, ksub); break;
  }
  return hipGetLastError();
}

template <bool PAGED>
hipError_t launch_generic(const PrefillArgs& a, DType dt, int head_dim, hipStream_t s) {
  if (a.num_seqs == 0 || a.max_seqlen == 0) return hipSuccess;
  const int group = a.num_q_heads / a.num_kv_heads;
  const dim3 grid(static_cast<unsigned>((a.max_seqlen + 3) / 4), static_cast<unsigned>(a.num_q_heads),
                  static_cast<unsigned>(a.num_seqs));
  if (dt == DType::BF16) {
    if (head_dim == 64) hipLaunchKernelGGL((prefill_generic_kernel<true, 64, PAGED>), grid, dim3(256), 0, s, a, group);
    else if (head_dim == 128) hipLaunchKernelGGL((prefill_generic_kernel<true, 128, PAGED>), grid, dim3(256), 0, s, a, group);
    else return hipErrorNotSupported;
  } else {
    if (head_dim == 64) hipLaunchKernelGGL((prefill_generic_kernel<false, 64, PAGED>), grid, dim3(256), 0, s, a, group);
    else if (head_dim == 128) hipLaunchKernelGGL((prefill_generic_kernel<false, 128, PAGED>), grid, dim3(256), 0, s, a, group);
    else return hipErrorNotSupported;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, DType dt, int head_dim, hipStream_t s) {
  if (a.num_seqs == 0 || a.max_seqlen == 0) return hipSuccess;
  if (dt == DType::BF16 && head_dim == kD) return launch_mfma<false>(a, a.num_q_heads / a.num_kv_heads, s);
  return launch_generic<false>(a, dt, head_dim, s);
}

hipError_t launch_prefill_generic(const PrefillArgs& a, DType dt, int head_dim, hipStream_t s) {
  return launch_generic<false>(a, dt, head_dim, s);
}

hipError_t launch_paged_prefill(const PrefillArgs& a, DType dt, int head_dim, hipStream_t s) {
  if (a.num_seqs == 0 || a.max_seqlen == 0) return hipSuccess;
  if (dt == DType::BF16 && head_dim == kD) return launch_mfma<true>(a, a.num_q_heads / a.num_kv_heads, s);
  return launch_generic<true>(a, dt, head_dim, s);
}

hipError_t launch_paged_prefill_generic(const PrefillArgs& a, DType dt, int head_dim, hipStream_t s) {
  return launch_generic<true>(a, dt, head_dim, s);
}

}  // namespace pa
