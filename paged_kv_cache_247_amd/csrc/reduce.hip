// Merge of split-context partitions. Each partition p of a (sequence, head) carries its max
// logit m_p, its exp-sum l_p and its normalised output o_p; with M = max_p m_p and
// w_p = l_p exp(m_p - M), the whole-context output is sum_p w_p o_p / sum_p w_p. This is an
// exact rewriting of the softmax sum (the pages describe no partitioning; it is how one long
// context is spread over many workgroups).
#include <limits.h>

#include "kernels.hpp"

namespace pkv {
namespace {

template <Dt DT, int D>
__global__ void __launch_bounds__(64) reduce_kernel(const ReduceParams a) {
  using T = typename Elt<DT>::T;
  constexpr int PER = D / 64;  // output columns per lane
  constexpr int U = 8;         // partition rows in flight
  const int H = a.num_heads;
  const int i = blockIdx.x / H;
  const int h = blockIdx.x % H;
  const int lane = lane_id();
  T* o = reinterpret_cast<T*>(a.out) + ((size_t)i * H + h) * D;

  const int L = max(a.context_lens[i], 0);
  const int n = min((int)(((int64_t)L + a.partition_size - 1) / a.partition_size),
                    a.max_num_partitions);
  if (n <= 0) {
#pragma unroll
    for (int e = 0; e < PER; ++e) o[lane + 64 * e] = from_f32<DT>(0.0f);
    return;
  }
  const size_t rec0 = ((size_t)i * H + h) * a.max_num_partitions;
  const float* ml = a.max_logits + rec0;
  const float* es = a.exp_sums + rec0;
  const float* to = a.tmp_out + rec0 * D + lane;

  // Lane p handles partition p (of each group of 64): M and the weight total first.
  float M = -INFINITY;
  for (int p = lane; p < n; p += 64) M = fmaxf(M, ml[p]);
  M = group_reduce<64>(M, OpMax());
  float den = 0.0f;
  for (int p = lane; p < n; p += 64) den += es[p] * __builtin_amdgcn_exp2f((ml[p] - M) * kLog2e);
  den = group_reduce<64>(den, OpAdd());

  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.0f;
  for (int p0 = 0; p0 < n; p0 += 64) {
    const int cnt = min(64, n - p0);
    // Normalised weight of this lane's partition; w / den is exactly 1 for a lone partition.
    float w = 0.0f;
    if (lane < cnt) w = es[p0 + lane] * __builtin_amdgcn_exp2f((ml[p0 + lane] - M) * kLog2e) / den;
    const float* row = to + (size_t)p0 * D;
    int p = 0;
    for (; p + U <= cnt; p += U) {
      float t[U][PER];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < PER; ++e) t[u][e] = row[(size_t)(p + u) * D + 64 * e];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float wp = bits_f((uint32_t)__builtin_amdgcn_readlane((int)f_bits(w), p + u));
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] = fmaf(wp, t[u][e], acc[e]);
      }
    }
    for (; p < cnt; ++p) {
      const float wp = bits_f((uint32_t)__builtin_amdgcn_readlane((int)f_bits(w), p));
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] = fmaf(wp, row[(size_t)p * D + 64 * e], acc[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < PER; ++e) o[lane + 64 * e] = from_f32<DT>(acc[e]);
}

template <Dt DT>
hipError_t launch_t(int head_dim, const ReduceParams& p, hipStream_t stream) {
  const dim3 grid((unsigned)p.num_seqs * p.num_heads);
  switch (head_dim) {
    case 64: reduce_kernel<DT, 64><<<grid, 64, 0, stream>>>(p); break;
    case 128: reduce_kernel<DT, 128><<<grid, 64, 0, stream>>>(p); break;
    default: return hipErrorNotSupported;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_reduce(Dt dt, int head_dim, const ReduceParams& p, hipStream_t stream) {
  switch (dt) {
    case Dt::F32: return launch_t<Dt::F32>(head_dim, p, stream);
    case Dt::F16: return launch_t<Dt::F16>(head_dim, p, stream);
    case Dt::BF16: return launch_t<Dt::BF16>(head_dim, p, stream);
  }
  return hipErrorNotSupported;
}

}  // namespace pkv
