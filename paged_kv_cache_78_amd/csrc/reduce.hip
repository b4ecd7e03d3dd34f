// Merge of split-context partials.
//
// A partition p of a (sequence, head) carries m_p (max of the scaled logits,
// natural-log units), l_p = sum exp(x_t - m_p) and the normalised partial
// output o_p.  Writing the design page's softmax definition ("Paged
// Attention", section "Softmax") over the union of disjoint token sets gives
//   M = max_p m_p,  w_p = l_p exp(m_p - M),  out = sum_p (w_p / sum_q w_q) o_p.
// The weights are normalised before they multiply o_p, so a single partition
// returns o_0 unchanged (weight exactly 1).
//
// One 64-lane workgroup per (sequence, head): lanes stride over partitions
// for the max and the weights (kept in LDS), then over head dims for the
// weighted sum, reading each o_p row as one coalesced load.
#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {
namespace {

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

template <typename OT, int D>
__global__ __launch_bounds__(64) void reduce_kernel(const ReduceParams p) {
  extern __shared__ float s_w[];   // [max_num_partitions]
  const int lane = threadIdx.x;
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  const int row = s * p.num_heads + h;
  const int NPM = p.max_num_partitions;
  const int L = p.context_lens[s];
  const int nps = L > 0 ? (L + p.partition_size - 1) / p.partition_size : 0;
  constexpr int PER = D / 64;      // head dims per lane
  uint16_t* out = reinterpret_cast<uint16_t*>(p.out) + (int64_t)row * D;

  if (L < 0 || nps > NPM || nps == 0) {
    const float v = (L == 0) ? 0.0f : __builtin_nanf("");
#pragma unroll
    for (int j = 0; j < PER; ++j) out[lane * PER + j] = to_bits16<OT>(v);
    return;
  }
  const float* ml = p.max_logits + (int64_t)row * NPM;
  const float* es = p.exp_sums + (int64_t)row * NPM;

  float mx = -__builtin_huge_valf();
  bool nan_seen = false;
  for (int i = lane; i < nps; i += 64) {
    const float v = ml[i];
    nan_seen |= (v != v);
    mx = fmaxf(mx, v);
  }
  mx = wave_max(mx);
  float tot = 0.0f;
  for (int i = lane; i < nps; i += 64) {
    const float w = es[i] * exp2_hw((ml[i] - mx) * kLog2e);
    s_w[i] = w;
    tot += w;
  }
  tot = wave_sum(tot);
  if (__builtin_amdgcn_ballot_w64(nan_seen) != 0) tot = __builtin_nanf("");
  for (int i = lane; i < nps; i += 64) s_w[i] = s_w[i] / tot;
  __syncthreads();

  const float* base = p.tmp_out + (int64_t)row * NPM * D + lane * PER;
  float acc[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) acc[j] = 0.0f;
  for (int i = 0; i < nps; ++i) {
    const float w = s_w[i];
    const float* src = base + (int64_t)i * D;
    if constexpr (PER == 2) {
      const float2_t v = *reinterpret_cast<const float2_t*>(src);
      acc[0] = fmaf(w, v[0], acc[0]);
      acc[1] = fmaf(w, v[1], acc[1]);
    } else {
      acc[0] = fmaf(w, src[0], acc[0]);
    }
  }
#pragma unroll
  for (int j = 0; j < PER; ++j) out[lane * PER + j] = to_bits16<OT>(acc[j]);
}

template <typename OT, int D>
hipError_t launch(const ReduceParams& p, hipStream_t stream) {
  dim3 grid(p.num_heads, p.num_seqs);
  const size_t lds = (size_t)(p.max_num_partitions > 0 ? p.max_num_partitions : 1) * sizeof(float);
  hipLaunchKernelGGL((reduce_kernel<OT, D>), grid, dim3(64), lds, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_reduce(const ReduceParams& p, Dt out_dt, int head_size, hipStream_t stream) {
  if (out_dt == Dt::F16) return head_size == 64 ? launch<F16, 64>(p, stream) : launch<F16, 128>(p, stream);
  return head_size == 64 ? launch<BF16, 64>(p, stream) : launch<BF16, 128>(p, stream);
}

}  // namespace pa
