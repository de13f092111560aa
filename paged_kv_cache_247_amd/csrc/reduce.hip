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

  // The records of the first 64 partitions and the first U partial rows lie inside the
  // workspace whatever the length, so they are loaded together with it: the wave waits for
  // memory once instead of once per step. Entries past the sequence's last partition are
  // never used.
  const size_t rec0 = ((size_t)i * H + h) * a.max_num_partitions;
  const float* ml = a.max_logits + rec0;
  const float* es = a.exp_sums + rec0;
  const float* to = a.tmp_out + rec0 * D + lane;
  const int pre = min(64, a.max_num_partitions);
  float ml0 = -INFINITY, es0 = 0.0f;
  if (lane < pre) {
    ml0 = ml[lane];
    es0 = es[lane];
  }
  float t0[U][PER];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int e = 0; e < PER; ++e) t0[u][e] = u < pre ? to[(size_t)u * D + 64 * e] : 0.0f;

  const int L = max(a.context_lens[i], 0);
  const int n = min((int)(((int64_t)L + a.partition_size - 1) / a.partition_size),
                    a.max_num_partitions);
  if (n <= 0) {
#pragma unroll
    for (int e = 0; e < PER; ++e) o[lane + 64 * e] = from_f32<DT>(0.0f);
    return;
  }

  float M = lane < n ? fmaxf(-INFINITY, ml0) : -INFINITY;
  for (int p = lane + 64; p < n; p += 64) M = fmaxf(M, ml[p]);
  M = group_reduce<64>(M, OpMax());
  float den = lane < n ? es0 * __builtin_amdgcn_exp2f((ml0 - M) * kLog2e) : 0.0f;
  for (int p = lane + 64; p < n; p += 64) den += es[p] * __builtin_amdgcn_exp2f((ml[p] - M) * kLog2e);
  den = group_reduce<64>(den, OpAdd());

  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.0f;
  for (int p0 = 0; p0 < n; p0 += 64) {
    const int cnt = min(64, n - p0);
    float w = 0.0f;
    if (lane < cnt)
      w = p0 == 0 ? es0 * __builtin_amdgcn_exp2f((ml0 - M) * kLog2e) / den
                  : es[p0 + lane] * __builtin_amdgcn_exp2f((ml[p0 + lane] - M) * kLog2e) / den;
    const float* row = to + (size_t)p0 * D;
    int p = 0;
    if (p0 == 0) {  // the rows loaded up front
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (u < cnt) {
          const float wp = bits_f((uint32_t)__builtin_amdgcn_readlane((int)f_bits(w), u));
#pragma unroll
          for (int e = 0; e < PER; ++e) acc[e] = fmaf(wp, t0[u][e], acc[e]);
        }
      }
      p = min(U, cnt);
    }
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
