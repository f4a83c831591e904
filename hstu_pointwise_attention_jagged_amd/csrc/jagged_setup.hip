// Set-up kernels of the jagged attention: the per-block key timestamp ranges that the
// attention kernel's bias classification reads, and the longest-first work list of
// (sequence, query tile) items ("Actions Speak Louder than Words" as retold on
// chenhuiyu.github.io, section "另外三块拼图", item 1: jagged batches at their true lengths).
#include "common.h"
#include "kernels.h"

namespace hstu {

namespace {

constexpr int kBN = kAttnBlockN;  // keys per attention tile

// ------------------------------------------------------------------------------------
// Timestamp range of each 32-key block of each sequence: for block j of sequence b (keys
// 32 j .. min(32 j + 32, n) - 1 from the sequence start s0), stat[s0 + 32 j] = (min, max)
// of their timestamps.  Only these block-start entries are written; the attention kernel
// reads no other.  One thread per block: grid (blocks of the longest sequence / 256, B).
// ------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void block_stats_kernel(const int32_t *__restrict__ ts,
                                                          const int32_t *__restrict__ offsets,
                                                          int2 *__restrict__ stat) {
  const int b = blockIdx.y;
  const int s0 = offsets[b], n = offsets[b + 1] - s0;
  const int k0 = (blockIdx.x * 256 + threadIdx.x) * 32;
  if (k0 >= n) return;
  const int e = min(k0 + 32, n);
  int32_t mn = ts[s0 + k0], mx = mn;
  for (int j = k0 + 1; j < e; ++j) {
    const int32_t v = ts[s0 + j];
    mn = min(mn, v);
    mx = max(mx, v);
  }
  stat[s0 + k0] = int2{mn, mx};
}

// ------------------------------------------------------------------------------------
// Jagged schedule: one workgroup builds the (sequence, q-tile) list, ordered by the
// number of key tiles each item visits, largest first, with a counting sort.
// ------------------------------------------------------------------------------------
constexpr int kSchedThreads = 1024;
constexpr int kSchedBins = 4096;

__device__ __forceinline__ int item_cost(int n, int n_p, int t, int mask, int bm) {
  const int q0 = t * bm;
  const int q_end = min(n, q0 + bm);
  const int own = mask == 0 ? q_end : q_end - q0;
  return (n_p + kBN - 1) / kBN + (own + kBN - 1) / kBN;
}

__global__ __launch_bounds__(kSchedThreads) void schedule_kernel(const int32_t *offsets,
                                                                 const int32_t *p_offsets,
                                                                 int B, int mask, int bm,
                                                                 int nbins, int32_t *work,
                                                                 int32_t *n_work) {
  __shared__ int bins[kSchedBins];
  __shared__ int total;
  const int tid = threadIdx.x;
  for (int i = tid; i < nbins; i += kSchedThreads) bins[i] = 0;
  __syncthreads();
  for (int b = tid; b < B; b += kSchedThreads) {
    const int n = offsets[b + 1] - offsets[b];
    const int n_p = p_offsets ? p_offsets[b + 1] - p_offsets[b] : 0;
    const int nq = (n + bm - 1) / bm;
    for (int t = 0; t < nq; ++t) atomicAdd(&bins[min(item_cost(n, n_p, t, mask, bm), nbins - 1)], 1);
  }
  __syncthreads();
  if (tid == 0) {  // exclusive scan, most expensive bin first
    int run = 0;
    for (int i = nbins - 1; i >= 0; --i) {
      const int c = bins[i];
      bins[i] = run;
      run += c;
    }
    total = run;
  }
  __syncthreads();
  for (int b = tid; b < B; b += kSchedThreads) {
    const int n = offsets[b + 1] - offsets[b];
    const int n_p = p_offsets ? p_offsets[b + 1] - p_offsets[b] : 0;
    const int nq = (n + bm - 1) / bm;
    for (int t = 0; t < nq; ++t) {
      const int pos = atomicAdd(&bins[min(item_cost(n, n_p, t, mask, bm), nbins - 1)], 1);
      work[2 * pos] = b;
      work[2 * pos + 1] = t;
    }
  }
  if (tid == 0) *n_work = total;
}

}  // namespace

// 128 query rows (4 waves) per workgroup at every length: two such workgroups share a CU,
// and since their barriers are independent, one's wait overlaps the other's work (measured
// faster than 8-wave groups at 8 x 8192 as well).
int attn_block_m(int max_seq_len) {
  (void)max_seq_len;
  return 128;
}

hipError_t launch_schedule(const int32_t *offsets, const int32_t *p_offsets, int B, int mask,
                           int max_seq_len, int max_prefix_len, int32_t *work, int32_t *n_work,
                           hipStream_t stream) {
  const int bm = attn_block_m(max_seq_len);
  const int64_t max_cost = (int64_t)(max_prefix_len + kBN - 1) / kBN + (max_seq_len + kBN - 1) / kBN + 1;
  const int nbins = (int)(max_cost < kSchedBins ? max_cost : kSchedBins);
  schedule_kernel<<<1, kSchedThreads, 0, stream>>>(offsets, p_offsets, B, mask, bm, nbins, work,
                                                   n_work);
  return hipGetLastError();
}

hipError_t launch_block_stats(const int32_t *ts, const int32_t *offsets, int B, int max_seq_len,
                              int2 *stat, hipStream_t stream) {
  if (B <= 0 || max_seq_len <= 0) return hipSuccess;
  const int blocks = (max_seq_len + 31) / 32;
  block_stats_kernel<<<dim3((blocks + 255) / 256, B), 256, 0, stream>>>(ts, offsets, stat);
  return hipGetLastError();
}


}  // namespace hstu
