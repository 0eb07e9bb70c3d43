// paged_attention_reduce: merge split-KV partitions by log-sum-exp.
//
// Each partition's (out, lse) pair is an exact summary of its keys: with
// M = max lse and w = exp(lse - M) the merged output is sum w*out / sum w and
// the merged lse is M + log(sum w).  The LSE output of the varlen call
// ("Llama 4 inference doubling (FlashAttention-3 + PagedAttention + vLLM)",
// section 2.4) is what makes the merge exact.
//
// Under a sliding window of W keys the merge covers partitions lo/P ..
// ceil(ctx/P)-1 only (lo = max(0, ctx - W)): the ones before hold no visible
// key and the decode call leaves them unwritten.
//
// General kernel: one workgroup per (sequence, query head).  Pass 1 finds M;
// pass 2 turns a chunk of partition lse values into weights held in LDS; pass
// 3 streams the partition outputs (each wave takes every fourth partition,
// each lane a pair of dims, 8 partitions in flight per wave) and the four
// waves meet in LDS.
#include "kernels.h"

namespace pa {

template <bool BF, int D>
__global__ __launch_bounds__(256) void reduce_kernel(ReduceArgs a) {
  constexpr int DPL = D / 64;  // dims per lane
  constexpr int CHUNK = 1024;
  __shared__ float sm_w[CHUNK];
  __shared__ float sm_red[4];
  __shared__ float sm_acc[4][D];

  const size_t row = blockIdx.x;  // b * H_q + h
  const int b = static_cast<int>(row / a.num_q_heads);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t ctx = max(a.context_lens[b], 0);
  const int64_t live = (ctx + a.partition_size - 1) / a.partition_size;
  const int64_t first = a.window > 0 ? max<int64_t>(0, ctx - a.window) / a.partition_size : 0;
  const int n = static_cast<int>(max<int64_t>(0, min<int64_t>(live, a.max_partitions) - first));
  const float* lse_row = a.part_lse + row * a.max_partitions + first;
  const float* out_row = a.part_out + (row * a.max_partitions + first) * D;

  float mx = kNegInf;
  for (int i = tid; i < n; i += 256) mx = fmaxf(mx, lse_row[i]);
  mx = group_allreduce<64>(mx, OpMax());
  if (lane == 0) sm_red[wave] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(sm_red[0], sm_red[1]), fmaxf(sm_red[2], sm_red[3]));
  __syncthreads();

  float acc[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] = 0.f;
  float wsum = 0.f;
  if (M != kNegInf) {
    for (int c0 = 0; c0 < n; c0 += CHUNK) {
      const int cn = min(CHUNK, n - c0);
      for (int i = tid; i < cn; i += 256) {
        const float w = fast_exp2((lse_row[c0 + i] - M) * kLog2e);
        sm_w[i] = w;
        wsum += w;
      }
      __syncthreads();
#pragma unroll 8
      for (int i = wave; i < cn; i += 4) {
        const float w = sm_w[i];
        const float* o = out_row + static_cast<size_t>(c0 + i) * D + lane * DPL;
        if constexpr (DPL == 2) {
          const float2 v = *reinterpret_cast<const float2*>(o);
          acc[0] = fmaf(w, v.x, acc[0]);
          acc[1] = fmaf(w, v.y, acc[1]);
        } else {
          acc[0] = fmaf(w, o[0], acc[0]);
        }
      }
      __syncthreads();
    }
  }
  wsum = group_allreduce<64>(wsum, OpSum());
  if (lane == 0) sm_red[wave] = wsum;
#pragma unroll
  for (int e = 0; e < DPL; ++e) sm_acc[wave][lane * DPL + e] = acc[e];
  __syncthreads();
  const float W = sm_red[0] + sm_red[1] + sm_red[2] + sm_red[3];
  for (int d = tid; d < D; d += 256) {
    float o = 0.f;
    if (M != kNegInf) o = (sm_acc[0][d] + sm_acc[1][d] + sm_acc[2][d] + sm_acc[3][d]) / W;
    if constexpr (BF) {
      static_cast<uint16_t*>(a.out)[row * D + d] = f32_to_bf16_bits(o);
    } else {
      static_cast<float*>(a.out)[row * D + d] = o;
    }
  }
  if (tid == 0) a.lse[row] = (M != kNegInf) ? M + __log2f(W) * kLn2 : kNegInf;
}

// Few partitions (at most 32): one wave per (sequence, head) issues every
// load it needs at once -- lane p reads partition p's lse, and each lane
// reads its D/64 dims of every live partition -- so the merge costs one
// memory round trip.  Weights are formed per partition from the lse held by
// lane p (v_readlane).
template <bool BF, int D, int MAXP>
__global__ __launch_bounds__(256) void reduce_small_kernel(ReduceArgs a) {
  constexpr int DPL = D / 64;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const size_t row = static_cast<size_t>(blockIdx.x) * 4 + wave;  // b * H_q + h
  if (row >= static_cast<size_t>(a.num_seqs) * a.num_q_heads) return;
  // (rows fit 32 bits: the call rejects more than INT32_MAX of them)
  const int b = static_cast<int>(static_cast<uint32_t>(row) / static_cast<uint32_t>(a.num_q_heads));
  float got_lse = kNegInf;
  float o[MAXP][DPL];
  // Load partitions first .. first + nl - 1 of this row.
  auto load = [&](int64_t first, int nl) {
    const float* lse_row = a.part_lse + row * a.max_partitions + first;
    const float* out_row = a.part_out + (row * a.max_partitions + first) * D + lane * DPL;
    got_lse = lane < nl ? lse_row[lane] : kNegInf;
#pragma unroll
    for (int p = 0; p < MAXP; ++p) {
#pragma unroll
      for (int e = 0; e < DPL; ++e) o[p][e] = 0.f;
      if (p < nl) {
        if constexpr (DPL == 2) {
          const float2 v = *reinterpret_cast<const float2*>(out_row + static_cast<size_t>(p) * D);
          o[p][0] = v.x;
          o[p][1] = v.y;
        } else {
          o[p][0] = out_row[static_cast<size_t>(p) * D];
        }
      }
    }
  };
  // Without a window the merge starts at partition 0, so its loads need not
  // wait for the context length: every allocated partition (up to MAXP) is
  // read at once and the ones past the sequence's end are masked below.  A
  // window's first partition depends on the context length.
  const bool nowin = a.window <= 0;
  if (nowin) load(0, static_cast<int>(min<int64_t>(a.max_partitions, MAXP)));
  const int64_t ctx = max(a.context_lens[b], 0);
  const int64_t first = nowin ? 0 : max<int64_t>(0, ctx - a.window) / a.partition_size;
  const int64_t live = min<int64_t>((ctx + a.partition_size - 1) / a.partition_size, a.max_partitions);
  const int n = static_cast<int>(min<int64_t>(max<int64_t>(0, live - first), MAXP));
  if (!nowin) load(first, n);
  const float my_lse = lane < n ? got_lse : kNegInf;
  const float M = group_allreduce<64>(my_lse, OpMax());
  float acc[DPL], wsum = 0.f;
#pragma unroll
  for (int e = 0; e < DPL; ++e) acc[e] = 0.f;
  if (M != kNegInf) {
#pragma unroll
    for (int p = 0; p < MAXP; ++p) {
      if (p < n) {
        const float lp = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_lse), p));
        const float w = fast_exp2((lp - M) * kLog2e);
        wsum += w;
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[e] = fmaf(w, o[p][e], acc[e]);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < DPL; ++e) {
    const float v = M != kNegInf ? acc[e] / wsum : 0.f;
    const size_t idx = row * D + lane * DPL + e;
    if constexpr (BF) {
      static_cast<uint16_t*>(a.out)[idx] = f32_to_bf16_bits(v);
    } else {
      static_cast<float*>(a.out)[idx] = v;
    }
  }
  if (lane == 0) a.lse[row] = (M != kNegInf) ? M + __log2f(wsum) * kLn2 : kNegInf;
}

namespace {

// Most partitions one (sequence, head) can merge: all of them, or under a
// window of W keys at most (W-1)/P + 2 (its first key can sit anywhere in the
// first one).
int64_t live_bound(const ReduceArgs& a) {
  int64_t n = a.max_partitions;
  if (a.window > 0 && (a.window - 1) / a.partition_size + 2 < n) n = (a.window - 1) / a.partition_size + 2;
  return n;
}

template <bool BF, int D>
hipError_t launch_small(const ReduceArgs& a, hipStream_t s) {
  const int64_t rows = static_cast<int64_t>(a.num_seqs) * a.num_q_heads;
  const dim3 grid(static_cast<unsigned>((rows + 3) / 4));
  const int64_t nb = live_bound(a);
  if (nb <= 8)
    hipLaunchKernelGGL((reduce_small_kernel<BF, D, 8>), grid, dim3(256), 0, s, a);
  else if (nb <= 16)
    hipLaunchKernelGGL((reduce_small_kernel<BF, D, 16>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((reduce_small_kernel<BF, D, 32>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_reduce(const ReduceArgs& a, DType dt, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(a.num_seqs) * a.num_q_heads));
  if (a.num_seqs == 0) return hipSuccess;
  if (live_bound(a) <= 32 && (a.head_dim == 64 || a.head_dim == 128)) {
    if (dt == DType::BF16)
      return a.head_dim == 128 ? launch_small<true, 128>(a, s) : launch_small<true, 64>(a, s);
    return a.head_dim == 128 ? launch_small<false, 128>(a, s) : launch_small<false, 64>(a, s);
  }
  if (dt == DType::BF16) {
    if (a.head_dim == 128) hipLaunchKernelGGL((reduce_kernel<true, 128>), grid, dim3(256), 0, s, a);
    else if (a.head_dim == 64) hipLaunchKernelGGL((reduce_kernel<true, 64>), grid, dim3(256), 0, s, a);
    else return hipErrorNotSupported;
  } else {
    if (a.head_dim == 128) hipLaunchKernelGGL((reduce_kernel<false, 128>), grid, dim3(256), 0, s, a);
    else if (a.head_dim == 64) hipLaunchKernelGGL((reduce_kernel<false, 64>), grid, dim3(256), 0, s, a);
    else return hipErrorNotSupported;
  }
  return hipGetLastError();
}

}  // namespace pa
