// Internal launchers of libhstu (C++ linkage, not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hstu {

enum Act { ACT_NONE = 0, ACT_SILU = 1 };

enum OutType { OUT_BF16 = 0, OUT_F16 = 1 };

// out[M][N] = act(A[M][K] . W[N][K]^T + bias[N]): bf16 inputs, fp32 accumulation, output
// bf16 or fp16 (saturated to the finite range).  Requires K % 64 == 0, N % 64 == 0.
hipError_t launch_gemm(const uint16_t *A, const uint16_t *W, const float *bias, uint16_t *out,
                       int M, int N, int K, Act act, OutType out_type, hipStream_t stream);

// Attention parameters (device pointers unless noted).
struct AttnArgs {
  const int32_t *offsets;   // [B+1]
  const int32_t *ts;        // [T] or nullptr
  const uint16_t *q, *k, *v;  // fp16
  int64_t stride;           // elements between rows of q/k/v
  const int32_t *p_offsets; // prefix [B+1] or nullptr
  const int32_t *p_ts;      // prefix timestamps or nullptr
  const uint16_t *pk, *pv;  // fp16
  int64_t p_stride;
  const float *rab_pos;     // [rab_heads][pos_buckets] or nullptr
  const float *rab_time;    // [rab_heads][time_buckets] or nullptr
  int pos_buckets, time_buckets, rab_per_head;
  float *out;               // [T][H*dv]
  int64_t out_stride;
  const int2 *kstat;        // [T] at each 32-key block start: (min, max) ts of the block
  const int2 *p_kstat;      // [T_p] same for prefix rows
  const int32_t *work;      // [2*cap] (b, q-tile) pairs, longest first
  const int32_t *n_work;    // [1]
  int num_heads;
  int mask;                 // 0 causal, 1 self-only
};

// Attention gradients (attention_bwd.hip), causal mask, no prefix.
struct AttnBwdArgs {
  const int32_t *offsets;     // [B+1]
  const int32_t *ts;          // [T] or nullptr
  const uint16_t *q, *k, *v;  // fp16 rows, `stride` elements apart
  int64_t stride;
  const float *d_out;         // upstream gradient of the attention output [T][H*dv]
  int64_t d_stride;
  uint16_t *d_h;              // workspace [T][H*dv]: d_out x 2^-e in fp16 (same stride)
  uint32_t *d_max;            // workspace [1]: bits of max |d_out| (e is its exponent)
  const int2 *stat;           // (min, max) timestamp of each 32-row block, when ts is set
  const float *rab_pos;       // [rab_heads][pos_buckets] or nullptr
  const float *rab_time;      // [rab_heads][time_buckets] or nullptr
  int pos_buckets, time_buckets, rab_per_head;
  float *dq, *dk, *dv;        // [T][H*dh] each
  int64_t g_stride;
  const int32_t *work;        // [2*cap] (b, 128-row tile) pairs
  const int32_t *n_work;      // [1]
  int num_heads;
};

// dQ, dK, dV for every row: the scaled fp16 copy of d_out, then two kernels over the
// schedule's (sequence, 128-row tile) list.  stat must be filled when ts is set.
hipError_t launch_attention_bwd(const AttnBwdArgs &a, int dh, int64_t cap, int64_t total_rows,
                                hipStream_t stream);

constexpr int kAttnBlockMMin = 128;  // query rows per workgroup: 128, or 256 for long rows
constexpr int kAttnBlockN = 64;      // keys per LDS stage

// Query rows per attention workgroup for a batch whose longest sequence is max_seq_len.
int attn_block_m(int max_seq_len);

// Work list capacity (items) for a batch of B sequences and T tokens (any block size).
inline int64_t attn_work_capacity(int64_t B, int64_t T) {
  return (T + kAttnBlockMMin - 1) / kAttnBlockMMin + B + 1;
}

// Builds the longest-first (sequence, q-tile) list into work[0 .. 2*cap) and n_work.
hipError_t launch_schedule(const int32_t *offsets, const int32_t *p_offsets, int B, int mask,
                           int max_seq_len, int max_prefix_len, int32_t *work, int32_t *n_work,
                           hipStream_t stream);

hipError_t launch_attention(const AttnArgs &a, int dh, int max_seq_len, int64_t cap,
                            hipStream_t stream);

// For each sequence and each 32-key block j of it: stat[s0 + 32 j] = (min, max) of the
// block's timestamps (other entries are not written).
hipError_t launch_block_stats(const int32_t *ts, const int32_t *offsets, int B, int max_seq_len,
                              int2 *stat, hipStream_t stream);

// G[T][HDV] = LayerNorm(O) * gamma + beta, times U (fp16 row of uvqk), as bf16.
hipError_t launch_norm_gate(const float *O, const uint16_t *U, int64_t u_stride,
                            const float *gamma, const float *beta, float eps, uint16_t *G,
                            int T, int HDV, hipStream_t stream);

// Stochastic Length over a raw jagged batch (stochastic_length.hip): new offsets and the
// raw indices of the kept tokens, plus (if given) their timestamps and feature rows.
// mode is [B] int32 scratch; T_upper bounds the new total (the raw total).
hipError_t launch_stochastic_length(const int32_t *off, const double *u_keep, const uint32_t *keys,
                                    int B, int T_upper, int L, double thr_num, int32_t *new_off,
                                    int32_t *mode,
                                    const int32_t *ts, int32_t *kept, int32_t *new_ts,
                                    const uint16_t *x, uint16_t *x_out, int64_t row_elems,
                                    hipStream_t stream);

}  // namespace hstu
