// Split-KV work units of the decode kernels (and of the paged stream probe,
// which walks the same units): the positions a (sequence, partition) covers
// and the balanced flat order of units.
#pragma once

#include <type_traits>

#include "kernels.h"

namespace pa {

// Positions lo .. ctx-1 are visible (lo > 0 only under a sliding window:
// the query at ctx-1 keeps its last `window` keys, "PageAttention +
// FlashAttention golden combination", section 4.1); blocks wholly before lo
// are never read.
struct Range {
  int ctx, lo, blk_lo, blk_hi;
};

__device__ __forceinline__ Range work_range(const DecodeArgs& a, int b, int part) {
  const int cap = min(a.max_context_len, a.max_blocks_per_seq * a.block_size);
  const int ctx = clampi(a.context_lens[b], 0, cap);
  const int nblk = (ctx + a.block_size - 1) / a.block_size;
  Range r;
  r.ctx = ctx;
  r.lo = a.window > 0 ? max(0, ctx - a.window) : 0;
  const int wblk = r.lo / a.block_size;
  if (a.partition_size > 0) {
    const int per = a.partition_size / a.block_size;
    r.blk_lo = max(part * per, wblk);
    r.blk_hi = min(nblk, part * per + per);
  } else {
    r.blk_lo = wblk;
    r.blk_hi = nblk;
  }
  return r;
}

// Partitions of a split launch that a sliding window leaves empty (wholly
// before the window's first key) are not written; the window-aware merge
// starts past them.

// Split-KV work unit u of a flat launch: the whole partitions of every
// sequence (sequence by sequence), then the partial ones.  Full units first
// keeps the long work at the head of the dispatch order, and a grid with no
// empty units in front lets every CU take an even share of the bytes.  Only
// partitions that hold a visible key are units: under a sliding window the
// live ones are lo/P .. ceil(ctx/P)-1, the full ones ceil(lo/P) .. ctx/P-1,
// and the partial ones (at most two) the first live one when lo is not
// aligned and the one holding ctx-1 when ctx is not.  One wave computes it
// (lane l scans sequences l*K .. l*K+K-1); returns b = -1 past the last unit.
// At most 64*16 sequences.
struct Unit {
  int b, part;
};

// Live and full partition ranges of one sequence.
struct PartSpan {
  int f0, f1;   // live:  f0 .. f1-1
  int c0, c1;   // full:  c0 .. c1-1 (empty when c1 <= c0)
};

__device__ __forceinline__ PartSpan part_span(int ctx, int window, int per) {
  const int lo = window > 0 ? max(0, ctx - window) : 0;
  PartSpan p;
  p.f0 = lo / per;
  p.f1 = (ctx + per - 1) / per;
  p.c0 = (lo + per - 1) / per;
  p.c1 = ctx / per;
  return p;
}

__device__ __forceinline__ Unit flat_unit(const DecodeArgs& a, int u) {
  const int lane = threadIdx.x & 63;
  const int B = a.num_seqs;
  const int per = a.partition_size;
  const int cap = min(a.max_context_len, a.max_blocks_per_seq * a.block_size);
  const int K = (B + 63) >> 6;
  int nf = 0, np = 0;
  for (int k = 0; k < K; ++k) {
    const int sq = lane * K + k;
    if (sq < B) {
      const PartSpan ps = part_span(clampi(a.context_lens[sq], 0, cap), a.window, per);
      const int full = max(0, ps.c1 - ps.c0);
      nf += full;
      np += max(0, ps.f1 - ps.f0) - full;
    }
  }
  // inclusive scans of the per-lane counts
  int sf = nf, sp = np;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int tf = __shfl_up(sf, d), tp = __shfl_up(sp, d);
    if (lane >= d) {
      sf += tf;
      sp += tp;
    }
  }
  const int F = __builtin_amdgcn_readlane(sf, 63), P = __builtin_amdgcn_readlane(sp, 63);
  const bool full = u < F;
  if (!full && u >= F + P) return Unit{-1, 0};
  const int v = full ? u : u - F;
  const int incl = full ? sf : sp;
  // the lane whose range holds unit v, and the units before it
  const int owner = __popcll(__builtin_amdgcn_ballot_w64(incl <= v));
  const int excl = owner > 0 ? __shfl(incl, owner - 1) : 0;
  int rem = v - excl;
  for (int k = 0; k < K; ++k) {
    const int sq = owner * K + k;
    const PartSpan ps = part_span(sq < B ? clampi(a.context_lens[sq], 0, cap) : 0, a.window, per);
    const int nfull = max(0, ps.c1 - ps.c0);
    const int n = full ? nfull : max(0, ps.f1 - ps.f0) - nfull;
    if (rem < n) {
      // partial units: the unaligned first live partition (if any), then the
      // one after the full range (or the second live one when none is full)
      const int first_partial = ps.f0 < ps.c0 ? 1 : 0;
      return Unit{sq, full ? ps.c0 + rem : (rem < first_partial ? ps.f0 : max(ps.c1, ps.c0))};
    }
    rem -= n;
  }
  return Unit{-1, 0};
}

// Wait until at most N vector-memory loads of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_waitcnt vmcnt(%0)" ::"i"(N) : "memory");
#endif
}

// s_waitcnt vmcnt(n) for a wave-uniform n, a multiple of 4 in [0, 4K].
template <int K>
__device__ __forceinline__ void wait_vmcnt_x4(int n) {
  if constexpr (K > 0) {
    if (n >= 4 * K) {
      wait_vmcnt<4 * K>();
      return;
    }
    wait_vmcnt_x4<K - 1>(n);
  } else {
    wait_vmcnt<0>();
  }
}

// f(std::integral_constant<int, k>) for k = K .. N-1, unrolled (compile-time
// indices, e.g. of LDS ring slots).
template <int K, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (K < N) {
    f(std::integral_constant<int, K>{});
    static_for<K + 1, N>(f);
  }
}

// Wait until at most `ahead` (<= AHEAD, wave-uniform) tiles of PER loads each
// are still in flight.
template <int PER, int AHEAD>
__device__ __forceinline__ void wait_tiles_ahead(int ahead) {
  if constexpr (AHEAD > 0) {
    if (ahead >= AHEAD) {
      wait_vmcnt<PER * AHEAD>();
      return;
    }
    wait_tiles_ahead<PER, AHEAD - 1>(ahead);
  } else {
    wait_vmcnt<0>();
  }
}

}  // namespace pa
