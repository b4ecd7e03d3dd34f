// Merge of split-context partials.
//
// A partition p of a (sequence, head) carries m_p (max of the scaled logits,
// natural-log units), l_p = sum exp(x_t - m_p) and the normalised partial
// output o_p.  Writing the design page's softmax definition ("Paged
// Attention", section "Softmax") over the union of disjoint token sets gives
//   M = max_p m_p,  w_p = l_p exp(m_p - M),  out = sum_p (w_p / sum_q w_q) o_p.
// The weights are normalised before they multiply o_p, so a single partition
// returns o_0 unchanged (weight exactly 1, the other terms exact zeros).
//
// One 256-thread workgroup per (sequence, head).  The threads first share
// the max and the weights (LDS), then thread t owns float4 column chunk
// t % (D/4) and every R-th partition starting at t / (D/4)
// (R = 256 / (D/4)), keeping several 16-byte loads in flight; an LDS pass
// adds the R partial sums of each chunk.
#include "pa_device.h"
#include "pa_kernels.h"

namespace pa {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float block_max(float x, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = x;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__device__ __forceinline__ float block_sum(float x, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = x;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

template <typename OT, int D>
__global__ __launch_bounds__(kThreads) void reduce_kernel(const ReduceParams p) {
  constexpr int CH = D / 4;              // float4 chunks per row
  constexpr int R = kThreads / CH;       // partitions in flight per step
  constexpr int UNROLL = 8;
  extern __shared__ float s_w[];         // [max_num_partitions] weights
  __shared__ float s_red[4];
  __shared__ float4_t s_part[kThreads];

  const int tid = threadIdx.x;
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  const int row = s * p.num_heads + h;
  const int NPM = p.max_num_partitions;
  const int L = p.context_lens[s];
  const int nps = L > 0 ? (L + p.partition_size - 1) / p.partition_size : 0;
  uint16_t* out = reinterpret_cast<uint16_t*>(p.out) + (int64_t)row * D;

  if (L < 0 || nps > NPM || nps == 0) {
    const float v = (L == 0) ? 0.0f : __builtin_nanf("");
    for (int d = tid; d < D; d += kThreads) out[d] = to_bits16<OT>(v);
    return;
  }
  const float* ml = p.max_logits + (int64_t)row * NPM;
  const float* es = p.exp_sums + (int64_t)row * NPM;

  float mx = -__builtin_huge_valf();
  int nan_seen = 0;
  for (int i = tid; i < nps; i += kThreads) {
    const float v = ml[i];
    nan_seen |= (v != v);
    mx = fmaxf(mx, v);
  }
  mx = block_max(mx, s_red);
  float tot = 0.0f;
  for (int i = tid; i < nps; i += kThreads) {
    const float w = es[i] * exp2_hw((ml[i] - mx) * kLog2e);
    s_w[i] = w;
    tot += w;
  }
  tot = block_sum(tot, s_red);
  nan_seen = __syncthreads_or(nan_seen);
  if (nan_seen) tot = __builtin_nanf("");
  for (int i = tid; i < nps; i += kThreads) s_w[i] = s_w[i] / tot;
  __syncthreads();

  const int chunk = tid % CH;
  const int first = tid / CH;
  const float* base = p.tmp_out + (int64_t)row * NPM * D + chunk * 4;
  float4_t acc = {0.f, 0.f, 0.f, 0.f};
  int i = first;
  for (; i + (UNROLL - 1) * R < nps; i += UNROLL * R) {
    float4_t v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u)
      v[u] = *reinterpret_cast<const float4_t*>(base + (int64_t)(i + u * R) * D);
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const float w = s_w[i + u * R];
      acc[0] = fmaf(w, v[u][0], acc[0]);
      acc[1] = fmaf(w, v[u][1], acc[1]);
      acc[2] = fmaf(w, v[u][2], acc[2]);
      acc[3] = fmaf(w, v[u][3], acc[3]);
    }
  }
  for (; i < nps; i += R) {
    const float4_t v = *reinterpret_cast<const float4_t*>(base + (int64_t)i * D);
    const float w = s_w[i];
    acc[0] = fmaf(w, v[0], acc[0]);
    acc[1] = fmaf(w, v[1], acc[1]);
    acc[2] = fmaf(w, v[2], acc[2]);
    acc[3] = fmaf(w, v[3], acc[3]);
  }
  s_part[tid] = acc;
  __syncthreads();
  if (tid < CH) {
    float4_t sum = s_part[tid];
    for (int r = 1; r < R; ++r) {
      const float4_t o = s_part[tid + r * CH];
      sum[0] += o[0];
      sum[1] += o[1];
      sum[2] += o[2];
      sum[3] += o[3];
    }
    const uint32_t w0 = (uint32_t)to_bits16<OT>(sum[0]) | ((uint32_t)to_bits16<OT>(sum[1]) << 16);
    const uint32_t w1 = (uint32_t)to_bits16<OT>(sum[2]) | ((uint32_t)to_bits16<OT>(sum[3]) << 16);
    *reinterpret_cast<u32x2_t*>(out + tid * 4) = u32x2_t{w0, w1};
  }
}

template <typename OT, int D>
hipError_t launch(const ReduceParams& p, hipStream_t stream) {
  dim3 grid(p.num_heads, p.num_seqs);
  const size_t lds = (size_t)(p.max_num_partitions > 0 ? p.max_num_partitions : 1) * sizeof(float);
  hipLaunchKernelGGL((reduce_kernel<OT, D>), grid, dim3(kThreads), lds, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_reduce(const ReduceParams& p, Dt out_dt, int head_size, hipStream_t stream) {
  if (out_dt == Dt::F16) return head_size == 64 ? launch<F16, 64>(p, stream) : launch<F16, 128>(p, stream);
  return head_size == 64 ? launch<BF16, 64>(p, stream) : launch<BF16, 128>(p, stream);
}

}  // namespace pa
