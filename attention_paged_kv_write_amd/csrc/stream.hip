// paged_kv_stream_read: the bandwidth ceiling of decode's memory access
// pattern.  Not a step of the method: it reads every K and V row a split-KV
// decode reads (the same work units in the same balanced flat order, the same
// 16-position tiles of one (block, KV head) slab) and does no attention, so
// its GB/s bounds what the decode kernels can reach with that pattern.
//
// Each wave folds the 32-bit words of the K and V rows of its unit's visible
// positions into one XOR checksum, so every byte it fetches is used and the
// result can be checked exactly against the pools.  Two ways to fetch:
//   DMA:  the decode kernel's own scheme, LDS-DMA (global_load_lds_dwordx4,
//         non-temporal) into a ring of DEPTH tile slots, DEPTH - 1 tiles in
//         flight while one is read back;
//   VGPR: plain non-temporal 16-byte loads into registers, DEPTH tiles issued
//         together before any is folded.
//
// pa_stream_read_contiguous: the plain ceiling beside it, a buffer read front
// to back (no table, no tiles), so that the paged pattern can be told from
// what HBM gives any read.
#include "kernels.h"
#include "units.h"

namespace pa {

namespace {

__device__ __forceinline__ uint32_t xor4(const u32x4 w) { return (w[0] ^ w[1]) ^ (w[2] ^ w[3]); }

// The eight 16-byte chunks this lane DMA'd into a ring slot (K rows, then V
// rows), then wait for them (inline asm, so the compiler adds no wait of its
// own for the LDS-DMA loads still in flight).
__device__ __forceinline__ void lds_read_slot8(u32x4* w, uint32_t addr) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile(
      "ds_read_b128 %0, %8\n\t"
      "ds_read_b128 %1, %8 offset:1024\n\t"
      "ds_read_b128 %2, %8 offset:2048\n\t"
      "ds_read_b128 %3, %8 offset:3072\n\t"
      "ds_read_b128 %4, %8 offset:4096\n\t"
      "ds_read_b128 %5, %8 offset:5120\n\t"
      "ds_read_b128 %6, %8 offset:6144\n\t"
      "ds_read_b128 %7, %8 offset:7168\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(w[0]), "=&v"(w[1]), "=&v"(w[2]), "=&v"(w[3]), "=&v"(w[4]), "=&v"(w[5]), "=&v"(w[6]),
        "=&v"(w[7])
      : "v"(addr)
      : "memory");
#else
  (void)w; (void)addr;
#endif
}

}  // namespace

// One wave per work unit (KV head, sequence, partition), bf16 rows of 128
// dims; BS = block size (a multiple of 16).
template <int BS, int DEPTH, bool DMA>
__global__ __launch_bounds__(64) void paged_stream_kernel(DecodeArgs a, uint32_t* sums) {
  constexpr int RC = 16;            // 16-byte chunks per 256-byte row
  constexpr int TPB = BS / 16;      // 16-position tiles per block
  __shared__ __attribute__((aligned(16))) u32x4 ring[DMA ? DEPTH : 1][DMA ? 512 : 1];

  int g, b, part;
  if (a.flat_units) {
    g = blockIdx.x % a.num_kv_heads;
    const Unit un = flat_unit(a, blockIdx.x / a.num_kv_heads);
    if (un.b < 0) return;
    b = __builtin_amdgcn_readfirstlane(un.b);
    part = __builtin_amdgcn_readfirstlane(un.part);
  } else {
    g = blockIdx.x;
    b = blockIdx.y;
    part = blockIdx.z;
  }
  const Range r = work_range(a, b, part);
  if (r.blk_lo >= r.blk_hi) return;
  const int lane = threadIdx.x & 63;
  const int j = lane >> 4, c16 = lane & 15;
  const int32_t* table = a.block_tables + static_cast<size_t>(b) * a.max_blocks_per_seq;
  const u32x4* kc = static_cast<const u32x4*>(a.k_cache);
  const u32x4* vc = static_cast<const u32x4*>(a.v_cache);
  const int n_blocks = r.blk_hi - r.blk_lo;
  uint32_t acc = 0;

  for (int w0 = 0; w0 < n_blocks; w0 += 64) {
    const int e = r.blk_lo + w0 + lane;
    const int ids = e < a.max_blocks_per_seq ? table[e] : -1;
    const int nt = min(64, n_blocks - w0) * TPB;
    // tile n: element offset of its first row in the pools, its first
    // position and the limit of valid positions (0 for a block id outside
    // the pool, a precondition violation: block 0 is read, nothing folded)
    auto tile = [&](int n, int& pos0, int& lim) -> size_t {
      int phys = __builtin_amdgcn_readlane(ids, n / TPB);
      const bool ok = phys >= 0 && phys < a.num_blocks;
      lim = ok ? r.ctx : 0;
      phys = ok ? phys : 0;
      pos0 = (r.blk_lo + w0 + n / TPB) * BS + (n % TPB) * 16;
      return ((static_cast<size_t>(phys) * a.num_kv_heads + g) * BS + (n % TPB) * 16) * RC;
    };
    // this lane's share of a tile: chunk c16 of rows 4c + j, K then V
    auto fold = [&](int pos0, int lim, const u32x4* w) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int pos = pos0 + 4 * c + j;
        if (pos < lim && pos >= r.lo) acc ^= xor4(w[c]) ^ xor4(w[4 + c]);
      }
    };
    if constexpr (DMA) {
      auto fetch = [&](int n) {
        int pos0, lim;
        const size_t base = tile(n, pos0, lim);
        u32x4* slot = ring[n % DEPTH];
#pragma unroll
        for (int c = 0; c < 4; ++c) global_to_lds16<2>(kc + base + (4 * c + j) * RC + c16, &slot[64 * c]);
#pragma unroll
        for (int c = 0; c < 4; ++c) global_to_lds16<2>(vc + base + (4 * c + j) * RC + c16, &slot[256 + 64 * c]);
      };
      for (int n = 0; n < DEPTH - 1 && n < nt; ++n) fetch(n);
      for (int n = 0; n < nt; ++n) {
        if (n + DEPTH - 1 < nt) fetch(n + DEPTH - 1);
        wait_tiles_ahead<8, DEPTH - 1>(min(DEPTH - 1, nt - 1 - n));
        u32x4 w[8];
        lds_read_slot8(w, lds_addr(&ring[n % DEPTH][lane]));
        int pos0, lim;
        tile(n, pos0, lim);
        fold(pos0, lim, w);
      }
    } else {
      for (int n0 = 0; n0 < nt; n0 += DEPTH) {
        u32x4 w[DEPTH][8];
#pragma unroll
        for (int t = 0; t < DEPTH; ++t) {
          if (n0 + t < nt) {
            int pos0, lim;
            const size_t base = tile(n0 + t, pos0, lim);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              w[t][c] = __builtin_nontemporal_load(kc + base + (4 * c + j) * RC + c16);
              w[t][4 + c] = __builtin_nontemporal_load(vc + base + (4 * c + j) * RC + c16);
            }
          }
        }
#pragma unroll
        for (int t = 0; t < DEPTH; ++t) {
          if (n0 + t < nt) {
            int pos0, lim;
            tile(n0 + t, pos0, lim);
            fold(pos0, lim, w[t]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(acc), m));
  if (lane == 0) sums[(static_cast<size_t>(b) * a.num_kv_heads + g) * a.num_partitions + part] = acc;
}

// Wave w (one per workgroup) reads 16-byte chunks [w * cpw, min((w + 1) * cpw,
// n)), lane l the chunks w * cpw + l + 64k, DEPTH non-temporal loads in flight
// per lane, and writes the XOR of their 32-bit words to sums[w].
template <int DEPTH>
__global__ __launch_bounds__(64) void contiguous_read_kernel(const u32x4* __restrict__ src, uint64_t n, uint64_t cpw,
                                                             uint32_t* sums) {
  const uint64_t w = blockIdx.x;
  const int lane = threadIdx.x;
  const uint64_t lo = w * cpw;
  const uint64_t hi = lo + cpw < n ? lo + cpw : n;
  uint32_t acc = 0;
  for (uint64_t base = lo + lane; base < hi; base += 64 * DEPTH) {
    u32x4 v[DEPTH];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const uint64_t idx = base + 64 * d;
      v[d] = idx < hi ? __builtin_nontemporal_load(src + idx) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) acc ^= xor4(v[d]);
  }
  for (int m = 32; m >= 1; m >>= 1) acc ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(acc), m));
  if (lane == 0) sums[w] = acc;
}

namespace {

template <int BS, int DEPTH, bool DMA>
hipError_t launch_stream_bd(const DecodeArgs& a, uint32_t* sums, hipStream_t s) {
  DecodeArgs f = a;
  const int64_t nwg = static_cast<int64_t>(a.num_kv_heads) * a.num_seqs * a.num_partitions;
  f.flat_units = a.num_seqs <= 64 * 16 && nwg * 64 <= 0xffffffffLL;
  const dim3 grid = f.flat_units ? dim3(static_cast<unsigned>(nwg))
                                 : dim3(static_cast<unsigned>(a.num_kv_heads), static_cast<unsigned>(a.num_seqs),
                                        static_cast<unsigned>(a.num_partitions));
  hipLaunchKernelGGL((paged_stream_kernel<BS, DEPTH, DMA>), grid, dim3(64), 0, s, f, sums);
  return hipGetLastError();
}

template <int BS>
hipError_t launch_stream_b(const DecodeArgs& a, uint32_t* sums, int depth, bool dma, hipStream_t s) {
  if (dma) {
    switch (depth) {
      case 2: return launch_stream_bd<BS, 2, true>(a, sums, s);
      case 3: return launch_stream_bd<BS, 3, true>(a, sums, s);
      case 4: return launch_stream_bd<BS, 4, true>(a, sums, s);
      default: return hipErrorNotSupported;
    }
  }
  switch (depth) {
    case 1: return launch_stream_bd<BS, 1, false>(a, sums, s);
    case 2: return launch_stream_bd<BS, 2, false>(a, sums, s);
    case 4: return launch_stream_bd<BS, 4, false>(a, sums, s);
    default: return hipErrorNotSupported;
  }
}

}  // namespace

hipError_t launch_contiguous_read(const void* src, uint64_t bytes, int waves, int depth, uint32_t* sums,
                                  hipStream_t s) {
  const uint64_t n = bytes / 16;
  const uint64_t cpw = (n + waves - 1) / waves;
  const u32x4* p = static_cast<const u32x4*>(src);
  switch (depth) {
    case 1: hipLaunchKernelGGL((contiguous_read_kernel<1>), dim3(waves), dim3(64), 0, s, p, n, cpw, sums); break;
    case 2: hipLaunchKernelGGL((contiguous_read_kernel<2>), dim3(waves), dim3(64), 0, s, p, n, cpw, sums); break;
    case 4: hipLaunchKernelGGL((contiguous_read_kernel<4>), dim3(waves), dim3(64), 0, s, p, n, cpw, sums); break;
    case 8: hipLaunchKernelGGL((contiguous_read_kernel<8>), dim3(waves), dim3(64), 0, s, p, n, cpw, sums); break;
    default: return hipErrorNotSupported;
  }
  return hipGetLastError();
}

hipError_t launch_stream(const DecodeArgs& a, uint32_t* sums, int depth, bool dma, hipStream_t s) {
  switch (a.block_size) {
    case 16: return launch_stream_b<16>(a, sums, depth, dma, s);
    case 32: return launch_stream_b<32>(a, sums, depth, dma, s);
    case 64: return launch_stream_b<64>(a, sums, depth, dma, s);
    default: return hipErrorNotSupported;
  }
}

}  // namespace pa
