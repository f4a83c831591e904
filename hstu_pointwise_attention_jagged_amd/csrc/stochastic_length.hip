// Stochastic Length: the per-user sequence subsampling applied to a raw jagged batch
// before the layer ("Actions Speak Louder than Words" as summarised on ltzyclt.github.io,
// section 5.1; chenhuiyu.github.io, section "另外三块拼图", item 2).
//
// For user b with n raw tokens, L = floor(N^(alpha/2)):
//   * the user keeps all n tokens when n <= L, or when its uniform draw u_b is below
//     N^alpha / n^2 (compared in fp64; the pages give that keep probability);
//   * otherwise it keeps L distinct positions chosen uniformly: the L tokens whose
//     (32-bit priority, position) pairs are smallest, in time order.
// The random numbers (u per user, one priority per raw token) are inputs, so the result
// is a deterministic function of them.
//
// gfx950 layout of the work
//  * sl_lengths_kernel (one workgroup): per-user decision and new length, then an
//    exclusive scan into the new offsets (one pass over the users per thread chunk).
//  * sl_select_kernel (one workgroup per user): a subsampled user's threshold pair is
//    found by an MSB-first radix select over the priorities (four 8-bit digit passes,
//    256-bin LDS histograms); the kept tokens are then compacted in time order with
//    wave ballots and a workgroup scan per 1024-token tile, which also ranks the tokens
//    that share the threshold priority by position.
//  * sl_gather_kernel (grid-stride over the whole GPU): timestamps and feature rows of
//    the kept tokens, in 16-byte copies; its length is the device-side new total, and
//    it is launched for the raw total as an upper bound.
#include "common.h"
#include "kernels.h"

namespace hstu {

namespace {

constexpr int kSlThreads = 1024;
constexpr int kSlWaves = kSlThreads / 64;

// Exclusive prefix over the workgroup of one value per thread; returns the prefix and
// writes the workgroup total to *total.  Uses ballots for 0/1 values.
__device__ __forceinline__ int block_excl_scan_flag(bool flag, int *wave_tot, int *total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t m = __ballot(flag);
  const uint64_t below = lane == 0 ? 0ull : (m & ((~0ull) >> (64 - lane)));
  const int in_wave = __popcll(below);
  if (lane == 0) wave_tot[wave] = __popcll(m);
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kSlWaves; ++w) {
    const int c = wave_tot[w];
    before += w < wave ? c : 0;
    all += c;
  }
  __syncthreads();  // wave_tot is reused by the next call
  *total = all;
  return before + in_wave;
}

__global__ __launch_bounds__(kSlThreads) void sl_lengths_kernel(const int32_t *__restrict__ off,
                                                                const double *__restrict__ u_keep,
                                                                int B, int L, double thr_num,
                                                                int32_t *__restrict__ new_off,
                                                                int32_t *__restrict__ mode) {
  __shared__ int wave_sum[kSlWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // contiguous chunk of users per thread
  const int per = (B + kSlThreads - 1) / kSlThreads;
  const int b0 = min(B, tid * per), b1 = min(B, b0 + per);
  int local = 0;
  for (int b = b0; b < b1; ++b) {
    const int n = off[b + 1] - off[b];
    const bool whole = n <= L || u_keep[b] < thr_num / ((double)n * (double)n);
    mode[b] = whole ? 0 : 1;
    local += whole ? n : L;
  }
  // workgroup exclusive scan of the per-thread sums
  int incl = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wave_sum[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += wave_sum[w];
  int run = before + incl - local;
  for (int b = b0; b < b1; ++b) {
    new_off[b] = run;
    const int n = off[b + 1] - off[b];
    run += mode[b] == 0 ? n : L;
  }
  if (tid == kSlThreads - 1) new_off[B] = run;
}

__global__ __launch_bounds__(kSlThreads) void sl_select_kernel(
    const int32_t *__restrict__ off, const uint32_t *__restrict__ keys, int L,
    const int32_t *__restrict__ new_off, const int32_t *__restrict__ mode,
    int32_t *__restrict__ kept) {
  __shared__ int hist[256];
  __shared__ int wave_tot[kSlWaves];
  __shared__ int sel[2];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int s0 = off[b], n = off[b + 1] - s0;
  const int o0 = new_off[b];
  const uint32_t *k = keys + s0;

  if (mode[b] == 0) {
    for (int i = tid; i < n; i += kSlThreads) kept[o0 + i] = s0 + i;
  } else {
    // radix select: the L-th smallest priority P, and how many tokens with priority P
    // are kept (the earliest ones)
    uint32_t prefix = 0, pmask = 0;
    int remaining = L;  // 1-based rank still to find among keys matching prefix
    for (int d = 3; d >= 0; --d) {
      for (int i = tid; i < 256; i += kSlThreads) hist[i] = 0;
      __syncthreads();
      const int sh = 8 * d;
      for (int i = tid; i < n; i += kSlThreads) {
        const uint32_t v = k[i];
        if ((v & pmask) == prefix) atomicAdd(&hist[(v >> sh) & 255u], 1);
      }
      __syncthreads();
      // the bin holding rank `remaining`: prefix sums over the 256 bins (four waves of
      // 64 bins), and the one thread whose bin covers the rank records it
      // (every thread passes both barriers; only the first four waves hold bins)
      const int lane = tid & 63, wave = tid >> 6;
      const int cnt = tid < 256 ? hist[tid] : 0;
      int incl = cnt;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o, 64);
        if (lane >= o) incl += v;
      }
      if (tid < 256 && lane == 63) wave_tot[wave] = incl;
      __syncthreads();
      if (tid < 256) {
        int before = 0;
        for (int w = 0; w < wave; ++w) before += wave_tot[w];
        const int excl = before + incl - cnt;
        if (cnt > 0 && excl < remaining && remaining <= excl + cnt) {
          sel[0] = tid;
          sel[1] = remaining - excl;
        }
      }
      __syncthreads();
      prefix |= (uint32_t)sel[0] << sh;
      pmask |= 255u << sh;
      remaining = sel[1];
      __syncthreads();  // sel and hist are rewritten by the next pass
    }
    const uint32_t P = prefix;
    const int need = remaining;  // kept tokens with priority P (>= 1)
    // compaction in time order, tile by tile
    int base_keep = 0, base_eq = 0;
    for (int t0 = 0; t0 < n; t0 += kSlThreads) {
      const int i = t0 + tid;
      const uint32_t v = i < n ? k[i] : 0xffffffffu;
      const bool is_eq = i < n && v == P;
      int tot_eq;
      const int eq_rank = base_eq + block_excl_scan_flag(is_eq, wave_tot, &tot_eq);
      const bool keep = i < n && (v < P || (is_eq && eq_rank < need));
      int tot_keep;
      const int pos = base_keep + block_excl_scan_flag(keep, wave_tot, &tot_keep);
      if (keep) kept[o0 + pos] = s0 + i;
      base_keep += tot_keep;
      base_eq += tot_eq;
    }
  }
}

constexpr int kGatherThreads = 256;

__global__ __launch_bounds__(kGatherThreads) void sl_gather_kernel(
    const int32_t *__restrict__ new_off, int B, const int32_t *__restrict__ kept,
    const int32_t *__restrict__ ts, int32_t *__restrict__ new_ts, const uint16_t *__restrict__ x,
    uint16_t *__restrict__ x_out, int64_t row_elems) {
  const int64_t T_new = new_off[B];
  const int64_t gid = (int64_t)blockIdx.x * kGatherThreads + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * kGatherThreads;
  if (new_ts != nullptr)
    for (int64_t r = gid; r < T_new; r += stride) new_ts[r] = ts[kept[r]];
  if (x_out != nullptr) {
    // 16-byte chunks: row_elems is a multiple of 8 (checked by the entry point)
    const int64_t cpr = row_elems / 8;
    const int64_t total = T_new * cpr;
    for (int64_t c = gid; c < total; c += stride) {
      const int64_t r = c / cpr;
      const int64_t e = (c - r * cpr) * 8;
      const int64_t src = (int64_t)kept[r] * row_elems + e;
      *reinterpret_cast<u32x4 *>(x_out + r * row_elems + e) =
          *reinterpret_cast<const u32x4 *>(x + src);
    }
  }
}

}  // namespace

hipError_t launch_stochastic_length(const int32_t *off, const double *u_keep, const uint32_t *keys,
                                    int B, int T_upper, int L, double thr_num, int32_t *new_off,
                                    int32_t *mode,
                                    const int32_t *ts, int32_t *kept, int32_t *new_ts,
                                    const uint16_t *x, uint16_t *x_out, int64_t row_elems,
                                    hipStream_t stream) {
  // (with B = 0 this only writes new_off[0] = 0)
  sl_lengths_kernel<<<1, kSlThreads, 0, stream>>>(off, u_keep, B, L, thr_num, new_off, mode);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || B == 0) return e;
  sl_select_kernel<<<B, kSlThreads, 0, stream>>>(off, keys, L, new_off, mode, kept);
  e = hipGetLastError();
  if (e != hipSuccess || (new_ts == nullptr && x_out == nullptr)) return e;
  // upper bound on the work: every raw token kept (rows of row_elems / 8 chunks)
  const int64_t per_row = x_out != nullptr ? row_elems / 8 : 1;
  const int64_t work = (int64_t)T_upper * per_row;
  const int64_t want = (work + kGatherThreads - 1) / kGatherThreads;
  const int grid = (int)(want < 1 ? 1 : (want > 8192 ? 8192 : want));
  sl_gather_kernel<<<grid, kGatherThreads, 0, stream>>>(new_off, B, kept, ts, new_ts, x, x_out,
                                                        row_elems);
  return hipGetLastError();
}

}  // namespace hstu
