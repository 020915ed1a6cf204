// Window recall of libsta: the share of full-attention probability that a
// candidate window keeps, averaged over the query rows of each (batch, head).
//
// For a query row i, sum_{j in window} softmax_full(i)_j equals
// exp(lse_window(i) - lse_full(i)), with lse the log-sum-exp of the row's
// scores over the window keys and over all keys. The attention kernels write
// both lse arrays; this kernel reduces them. One workgroup per (batch, head)
// walks its S rows in a fixed order and sums in double precision, so the
// result is deterministic.
#include <hip/hip_runtime.h>

#include "sta_kernels.h"

namespace sta {
namespace {

constexpr int kRecallThreads = 256;

__global__ void __launch_bounds__(kRecallThreads)
recall_reduce_kernel(const float* lse_full, const float* lse_win, float* recall, int S, int n_cand,
                     int c) {
  __shared__ double part[kRecallThreads / 64];
  const long long base = (long long)blockIdx.x * S;
  double acc = 0.0;
  for (int i = threadIdx.x; i < S; i += kRecallThreads)
    acc += (double)__expf(lse_win[base + i] - lse_full[base + i]);
  for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    double sum = 0.0;
    for (int w = 0; w < kRecallThreads / 64; ++w) sum += part[w];
    recall[(long long)blockIdx.x * n_cand + c] = (float)(sum / S);
  }
}

}  // namespace

int launch_recall_reduce(const float* lse_full, const float* lse_win, float* recall, int BH, int S,
                         int n_cand, int c, void* stream) {
  hipLaunchKernelGGL(recall_reduce_kernel, dim3((unsigned)BH), dim3(kRecallThreads), 0,
                     static_cast<hipStream_t>(stream), lse_full, lse_win, recall, S, n_cand, c);
  return (int)hipGetLastError();
}

}  // namespace sta
