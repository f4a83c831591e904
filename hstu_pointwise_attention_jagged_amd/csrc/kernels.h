// Internal launchers of libhstu (C++ linkage, not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hstu {

enum Act { ACT_NONE = 0, ACT_SILU = 1 };

enum OutType { OUT_BF16 = 0, OUT_F16 = 1, OUT_F32 = 2 };

// Operand layouts of the 256 x 256 GEMM: KC, rows are output rows (or columns) with K
// contiguous; KR, rows are K.
enum Layout { KC = 0, KR = 1 };

// C[M][N] = sum_k X(m, k) W(n, k) (+ bias[n], activation): X(m, k) = x[m ldx + k] (KC) or
// x[k ldx + m] (KR), likewise W with ldw.  With splits > 1, split s sums k in
// [s k_split, (s + 1) k_split) into its own [M][N] fp32 slice of out.
// The f2 operand conversion, w2 (bf16, n_w values) -> fp16 w2h and gamma / beta (fp32,
// either may be nullptr: 1 / 0) -> fp16 gb [2][K] when gb is not nullptr.  Given to the
// f1 launch_gemm, it runs as extra workgroups of the same launch (large tiles: they are
// dispatched after every tile of the product and finish in its tail) or as its own launch
// right after the product (small tiles).
struct W2Prep {
  const uint16_t *w2 = nullptr;
  int64_t n_w = 0;
  const float *gamma = nullptr, *beta = nullptr;
  int K = 0;
  uint16_t *w2h = nullptr;  // nullptr: nothing to convert
  _Float16 *gb = nullptr;
  int blocks = 0;     // set by the launcher: workgroups of the conversion
  int grid_gemm = 0;  // set by the launcher: workgroups below this one run the product
};

struct GemmArgs {
  const uint16_t *x;
  int64_t ldx;
  const uint16_t *w;
  int64_t ldw;
  const float *bias;        // [N] or nullptr
  void *out;
  const int32_t *m_dev;     // (device) rows present, or nullptr
  int M, N, K;
  int k_split, splits;
  int n_tiles_n, n_tiles_total;
  int xcd_n;                // set by the launcher: XCDs along the feature tiles
  W2Prep prep;              // f1 only: the f2 operand conversion as a side job
};

// Largest reduction width of launch_gemm: a 256-row operand panel (256 K bf16 values)
// stays addressable with 32-bit byte offsets.
constexpr int kGemmMaxK = 1 << 21;

// out[M][N] = act(A[M][K] . W[N][K]^T + bias[N]): bf16 inputs, fp32 accumulation, output
// bf16 or fp16 (saturated to the finite range).  Requires K % 64 == 0, N % 64 == 0.
// With m_dev (device), only rows below min(M, *m_dev) are computed and written: M is then
// a capacity and the true row count is read on the device.  With prep, the f2 operand
// conversion runs beside the product (see W2Prep).
hipError_t launch_gemm(const uint16_t *A, const uint16_t *W, const float *bias, uint16_t *out,
                       int M, int N, int K, Act act, OutType out_type, hipStream_t stream,
                       const int32_t *m_dev = nullptr, const W2Prep *prep = nullptr);

// Backward products with fp32 output, bf16 operands, fixed summation order:
// NN  out[M][N] = X[M][K] . W[K][N]     (X rows of ldx, W rows of ldw; K % 64 == 0)
// TN  out[M][N] = X[K][M]^T . W[K][N]   (the reduction over K = tokens runs in splits
//     whose [M][N] partials, in `partial`, are then added in split order; `partial`
//     holds gemm_tn_partial_bytes(M, N, K) bytes, 0 when one split suffices)
hipError_t launch_gemm_nn_f32(const uint16_t *X, int64_t ldx, const uint16_t *W, int64_t ldw,
                              float *out, int M, int N, int K, hipStream_t stream);
hipError_t launch_gemm_tn_f32(const uint16_t *X, int64_t ldx, const uint16_t *W, int64_t ldw,
                              float *out, int M, int N, int K, float *partial, hipStream_t stream);
size_t gemm_tn_partial_bytes(int M, int N, int K);

// f2 with the LayerNorm and the U gate of equation 3 formed in its operand staging:
// out[M][N] = G w^T + bias, G = ((o - mu) rstd gamma + beta) U per row, where o is given
// per head as c (standardised fp16, [M][K]) with stats (mean, biased variance) [M][H].
struct GateGemmArgs {
  const uint16_t *w;        // fp16 [N][K] (w2 converted by launch_gate_prep)
  const uint16_t *c;        // fp16 [M][K]
  const uint16_t *u;        // fp16 gate rows, pitch u_stride
  int64_t u_stride;
  const float2 *stats;      // [M][H]
  const _Float16 *gb;       // fp16 [2][K] gamma | beta, or nullptr (no affine)
  const float *bias;        // [N] or nullptr
  uint16_t *out;            // bf16 [M][N]
  const int32_t *m_dev;     // (device) true row count, or nullptr: M rows (else M is a capacity)
  int M, N, K, H, dv;
  float eps;
  int n_tiles_n, n_tiles_total;  // set by the launcher
};
// w2 (bf16, n_w values) -> fp16 w2h; gamma / beta (either may be nullptr) -> fp16 gb [2][K]
// when gb is not nullptr.
hipError_t launch_gate_prep(const uint16_t *w2, int64_t n_w, const float *gamma, const float *beta,
                            int K, uint16_t *w2h, uint16_t *gb, hipStream_t stream);
hipError_t launch_gate_gemm(const GateGemmArgs &a, bool affine, hipStream_t stream);

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
  float *out;               // [T][H*dv] raw aggregation (when cn is nullptr)
  int64_t out_stride;       // elements between rows of out / cn
  uint16_t *cn;             // or: [T][H*dv] fp16, each head's part standardised with
  float2 *stats;            //     its (mean, biased variance), stats [T][H]
  const int2 *kstat;        // [T] at each 32-key block start: (min, max) ts of the block
  const int2 *p_kstat;      // [T_p] same for prefix rows
  const int32_t *work;      // [2*cap] (b, q-tile) pairs, longest first
  const int32_t *n_work;    // [1]
  int num_heads;
  int mask;                 // 0 causal, 1 self-only
  // profiling only, or nullptr: workgroup w < kClockSlots adds the core-clock and the
  // 100 MHz real-time ticks of its lifetime to clk[2 w], clk[2 w + 1]
  uint64_t *clk;
};
constexpr int kClockSlots = 64;

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
  // Output form.  z == nullptr: fp32 dq, dk, dv (g_stride).  Otherwise the gradients of
  // the pre-activations: bf16 dz = grad * SiLU'(z) at row r, column off + h dh + c of z
  // and dz (pitch z_stride), with off = zq_off, zk_off, zv_off for Q, K, V.
  const uint16_t *z;
  uint16_t *dz;
  int64_t z_stride, zq_off, zk_off, zv_off;
  // Gradients of the bias tables (rab_part == nullptr: not formed): per-work-item bins
  // [H][rab_cap][pos_buckets + time_buckets], reduced into d_rab_pos [rows][pos_buckets]
  // and d_rab_time [rows][time_buckets] (either may be nullptr), rows = H when the
  // tables are per head, else 1.
  float *rab_part;
  int64_t rab_cap;
  float *d_rab_pos, *d_rab_time;
  // dS stored by the dK/dV kernel for the dQ kernel (ds_buf == nullptr: the dQ kernel forms
  // dS again).  Per head, each sequence's causal triangle of 32 x 32 blocks, block (qb, kb)
  // (kb <= qb) of sequence b at h ds_head_blocks + tri_base[b] + qb (qb + 1) / 2 + kb, each
  // block 2 KB of fp16 in the dK/dV kernel's register order: [half s][lane L][8], holding
  // dS of key L % 32 and query 8 (e / 4) + 4 (L / 32) + e % 4, e = 8 s + 0..7.
  // tri_base [B + 1] is formed on the device.
  uint16_t *ds_buf;
  uint16_t *ds_dump;  // 2 KB that skipped blocks write (never read)
  int64_t ds_head_blocks;
  int64_t *tri_base;
  int batch;
  const float *rab_pos;       // [rab_heads][pos_buckets] or nullptr
  const float *rab_time;      // [rab_heads][time_buckets] or nullptr
  int pos_buckets, time_buckets, rab_per_head;
  float *dq, *dk, *dv;        // [T][H*dh] each
  int64_t g_stride;
  const int32_t *work;        // [2*cap] (b, 128-row tile) pairs
  const int32_t *n_work;      // [1]
  int num_heads;
};

// Backward of LayerNorm + gate for every row (see layer_bwd.hip).
struct NormGateBwdArgs {
  const float *o;       // [T][hdv] attention output, or nullptr: then O = cn sqrt(var) + mean
  const uint16_t *cn;   //   per head, from the forward's standardised fp16 output cn [T][hdv]
  const float2 *stats;  //   and its (mean, biased variance) per row and head [T][hdv / dv]
  int dv;               //   (head width)
  const float *dg;      // [T][hdv] gradient of the gate product G
  const uint16_t *u;    // fp16 gate U, row pitch u_stride
  const uint16_t *zu;   // fp16 pre-activations of U, row pitch u_stride
  int64_t u_stride;
  const float *gamma, *beta;  // [hdv] or nullptr
  float eps;
  uint16_t *g;          // bf16 [T][hdv]: G = LayerNorm(O) U
  uint16_t *dzu;        // bf16 gate columns of dZ, row pitch dz_stride
  int64_t dz_stride;
  float *d_o;           // [T][hdv]: gradient of O
  float *part_gamma, *part_beta;  // [norm_gate_bwd_waves(T)][hdv] partial sums or nullptr
  int T, hdv;
};
constexpr int kNgWaves = 4096;  // most waves (and partial rows) of the norm-gate backward
int norm_gate_bwd_waves(int T);
hipError_t launch_norm_gate_bwd(const NormGateBwdArgs &a, hipStream_t stream);
hipError_t launch_silu_f16(const uint16_t *z, uint16_t *out, int64_t n, hipStream_t stream);
hipError_t launch_fill_zero(float *p, int64_t n, hipStream_t stream);  // a kernel, not a memset
hipError_t launch_cast_bf16(const float *src, uint16_t *dst, int64_t n, hipStream_t stream);
// out[c] = sum of column c of a [rows][cols] matrix (fp32, or bf16 when bf16), through
// n_parts partial rows in `partial` ([n_parts][cols]); fixed summation order.
hipError_t launch_colsum(const void *a, bool bf16, int rows, int cols, int64_t stride,
                         float *partial, int n_parts, float *out, hipStream_t stream);
hipError_t launch_sum_parts(const float *partial, int n_parts, int cols, float *out,
                            hipStream_t stream);

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
