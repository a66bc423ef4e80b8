// chunk_map.hip -- varlen chunk map of the chunked prefill, built on the device
// from cu_seqlens without a host round trip.
//
//   order[r]      sequence id of rank r, longest sequence first, ties by id
//                 (the prefill launches its longest recurrences first so they
//                 do not straggle)
//   chunk_off[n]  exclusive prefix sum of ceil(len_n / 64)
//   chunk_tab[c]  (sequence id, first token, token count) of chunk c; chunks
//                 restart at every sequence start, the last one of a sequence
//                 may be partial (1..64 tokens), empty sequences have none
// Pure integer work: the result is unique and must match bit for bit.
#include "common.h"
#include "launch.h"

namespace gdn {

namespace {

constexpr int kChunk = 64;
constexpr int kThreads = 256;
constexpr int kLdsOffsets = 4096;   // chunk offsets kept in LDS for the table's searches

// rank_i = #{ j : len_j > len_i  or  (len_j == len_i and j < i) }
__global__ __launch_bounds__(kThreads) void order_kernel(const int32_t* __restrict__ cu,
                                                         int n_seqs, int32_t* __restrict__ order) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i >= n_seqs) return;
  const int li = cu[i + 1] - cu[i];
  int rank = 0;
  for (int j = 0; j < n_seqs; ++j) {
    const int lj = cu[j + 1] - cu[j];
    rank += (lj > li) || (lj == li && j < i);
  }
  order[rank] = i;
}

// One work-group: block-wise exclusive scan of chunk counts, then the table.
__global__ __launch_bounds__(kThreads) void chunk_table_kernel(const int32_t* __restrict__ cu,
                                                               int n_seqs,
                                                               int32_t* __restrict__ chunk_off,
                                                               int32_t* __restrict__ chunk_tab) {
  __shared__ int32_t scan[kThreads];
  __shared__ int32_t carry;
  __shared__ int32_t offs[kLdsOffsets];
  __shared__ int32_t cus[kLdsOffsets + 1];
  const int tid = threadIdx.x;
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < n_seqs; base += kThreads) {
    const int n = base + tid;
    const int cnt = n < n_seqs ? (cu[n + 1] - cu[n] + kChunk - 1) / kChunk : 0;
    scan[tid] = cnt;
    __syncthreads();
    // Hillis-Steele inclusive scan
    for (int d = 1; d < kThreads; d <<= 1) {
      const int add = tid >= d ? scan[tid - d] : 0;
      __syncthreads();
      scan[tid] += add;
      __syncthreads();
    }
    const int c0 = carry;
    if (n < n_seqs) chunk_off[n] = c0 + scan[tid] - cnt;
    __syncthreads();
    if (tid == kThreads - 1) carry = c0 + scan[tid];
    __syncthreads();
  }
  if (tid == 0) chunk_off[n_seqs] = carry;
  __syncthreads();
  // table: the threads take the chunks in turn; chunk c belongs to the
  // sequence n with chunk_off[n] <= c < chunk_off[n + 1] (binary search;
  // empty sequences own no chunk), so a long sequence is not one thread's loop
  // (the offsets searched in LDS when they fit)
  const int total = carry;
  const bool in_lds = n_seqs <= kLdsOffsets;
  if (in_lds) {
    for (int n = tid; n < n_seqs; n += kThreads) offs[n] = chunk_off[n];
    for (int n = tid; n <= n_seqs; n += kThreads) cus[n] = cu[n];
  }
  __syncthreads();
  const int32_t* off = in_lds ? offs : chunk_off;
  const int32_t* cuv = in_lds ? cus : cu;
  for (int c = tid; c < total; c += kThreads) {
    int lo = 0, hi = n_seqs - 1;          // largest n with off[n] <= c
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (off[mid] <= c) lo = mid; else hi = mid - 1;
    }
    const int s = cuv[lo];
    const int len = cuv[lo + 1] - s;
    const int t = (c - off[lo]) * kChunk;
    chunk_tab[3 * c + 0] = lo;
    chunk_tab[3 * c + 1] = s + t;
    chunk_tab[3 * c + 2] = min(kChunk, len - t);
  }
}

}  // namespace

hipError_t launch_chunk_map(const int32_t* cu, int n_seqs, int T_total, int32_t* order,
                            int32_t* chunk_off, int32_t* chunk_tab, hipStream_t stream) {
  (void)T_total;
  if (n_seqs > 0) {
    hipLaunchKernelGGL(order_kernel, dim3((n_seqs + kThreads - 1) / kThreads), dim3(kThreads), 0,
                       stream, cu, n_seqs, order);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(kThreads), 0, stream, cu, n_seqs,
                     chunk_off, chunk_tab);
  return hipGetLastError();
}

}  // namespace gdn
