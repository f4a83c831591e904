// Gradients of the jagged pointwise attention (equation 2 of the layer, "Actions Speak
// Louder than Words" as retold on chenhuiyu.github.io, section "HSTU Layer 到底改了什么"),
// causal mask, no prefix.  Per sequence and head, with S = Q K^T + rab^{p,t},
// A = SiLU(S) on allowed pairs and the upstream gradient dO of O = A V:
//
//   dA = dO V^T,  dS = dA * SiLU'(S) (0 on masked pairs),  dQ = dS K,  dK = dS^T Q,
//   dV = A^T dO,  SiLU'(x) = sigma(x) (1 + x (1 - sigma(x))).
//
// No softmax, so no row statistics: each gradient is a plain sum over pairs.  dQ, dK and
// dV are computed without atomics (fixed summation orders); the bias tables' sums add
// into per-wave LDS bins with LDS atomics, where only the lanes of one wave meet at an
// address.  The launches:
//  * prep: max |dO| over the batch, then dO x 2^-e in fp16, with 2^e the power of two
//    that brings that maximum into [0.5, 1).  Every gradient is linear in dO, so the
//    kernels multiply their results by 2^e (exact); tiny training gradients keep their
//    fp16 precision and dA, dS stay far from the fp16 range limit.
//  * attn_bwd_dkv_kernel: a workgroup of 4 waves owns 128 key rows (K fragments in
//    registers, V rows in LDS) and streams 32-query tiles of Q and dO.  Per 32 x 32 block:
//    S = Q K^T and dA = dO V^T (each lane holds 16 queries of one key), A and dS
//    elementwise, then dV^T += dO^T A and dK^T += Q^T dS through transposing LDS reads of Q
//    and dO.  When the workspace holds it, each block of dS is also stored (fp16).
//  * attn_bwd_dq_ds_kernel (dS stored): a workgroup owns 128 query rows and streams K tiles
//    and the stored dS blocks through LDS; per block dQ^T += K^T dS^T, both operands by the
//    transposing read.  The five products of the gradient each run once.
//  * attn_bwd_dq_kernel (dS not stored): a workgroup owns 128 query rows (Q and dO
//    fragments in registers) and streams key tiles of K and V.  Per block: S^T = K Q^T and
//    dA^T = V dO^T (each lane holds 16 keys of one query), dS^T elementwise, then
//    dQ^T += K^T dS^T: S and dA are formed a second time.
//  * the dQ kernels also sum dS per bias bucket when the tables' gradients are asked for;
//    rab_reduce_kernel adds the workgroups' sums in a fixed order.
// The kernels load the next tile into registers while the current one is computed.  The
// bias of a 32 x 32 block is classified once per wave from the blocks' timestamp ranges
// and position gap (the log2 time bucket is monotone in the gap): one value for the whole
// block (CONST), two values split by a time threshold (TWO), or per element (GENERAL,
// only near the diagonal or across several time buckets).  Operands are fp16 (Q, K, V
// as the forward takes them; dO, A and dS rounded to fp16), accumulation fp32.
#include <stdint.h>

#include "common.h"
#include "kernels.h"

namespace hstu {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kOwnRows = 32 * kWaves;  // rows a workgroup owns: the schedule's tile
// keys per tile streamed by the dQ kernel (32 at DH = 128, where the prefetch registers
// of a 64-key tile would not fit beside the wave's Q and dO fragments)
template <int DH>
constexpr int dq_keys() { return DH == 128 ? 32 : 64; }
constexpr int kDkvQueries = 32;        // queries per tile streamed by the dK/dV kernel
constexpr int kMaxPos = 1024;
constexpr int kMaxTime = 64;
constexpr int kTimeReps = 16;                   // copies of a wave's time bins
constexpr int kTimeRepPitch = kMaxTime + 1;     // so that copy r starts r banks further
constexpr float kNegLog2e = -1.4426950408889634f;

enum BlockKind { KIND_CONST = 0, KIND_TWO = 1, KIND_GENERAL = 2 };

// ds_read_b64_tr_b16: in each 16-lane group, lane 4 j + q gives the address of row j at
// features 4 q .. 4 q + 3 of a 16-feature slice and receives rows 0..3 of feature lane % 16
__device__ __forceinline__ u32x2 tr_read(const unsigned char *p) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  return __builtin_bit_cast(
      u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)p));
}

// LDS pitches: row copies (16-byte fragment reads of one chunk across 32 rows) and
// transposed-read copies.  LDS has 64 four-byte banks and a transposing read serves 32
// lanes at a time: 4 rows x 64 bytes, so the rows' pitch must step 16 banks (mod 64) for
// the 4 rows to fall on distinct banks (a pitch of 16 banks plus a multiple of 64).
template <int DH>
struct BwdLayout {
  static constexpr int ROWP = DH * 2 + 16;
  static constexpr int TRP = DH * 2 + (DH == 32 ? 0 : 64);
  static_assert((TRP / 4) % 64 == 16 || (TRP / 4) % 64 == 48, "transposed-read pitch");
  static constexpr int KS = DH / 16;   // k-steps over the head dimension
  static constexpr int FT = DH / 32;   // 32-wide feature tiles
  static constexpr int CPR = DH / 8;   // 16-byte chunks per row
};

// Buffer resource over the DH-wide head slice of rows [0, n) of one sequence (row pitch
// `stride` elements, first row at base): loads past the last row return zero, so a tile
// that runs past the sequence end needs no branch.  The host keeps the byte count below
// 2^31 (max_seq_len + 64 rows of the pitch).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const uint16_t *base, int64_t stride,
                                                            int n, int dh) {
  const uint32_t bytes = n > 0 ? (uint32_t)(((int64_t)(n - 1) * stride + dh) * 2) : 0u;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(base), 0, (int)bytes,
                                           0x00020000);  // raw buffer, 32-bit data format
}

// Load of a value that no thread writes while the kernel runs, through the constant
// address space: with a uniform address it becomes a scalar load.
template <class T>
__device__ __forceinline__ T ld_const(const T *ptr) {
  return *(const __attribute__((address_space(4))) T *)ptr;
}

// (min, max) timestamps of the 32-row block starting at row ptr - stat, as two scalar words
__device__ __forceinline__ int2 ld_stat(const int2 *ptr) {
  const int32_t *w = reinterpret_cast<const int32_t *>(ptr);
  return int2{ld_const(w), ld_const(w + 1)};
}

// Timestamps of rows [0, n) of one sequence, zero past the end (or everywhere without ts)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t ts_rsrc(const int32_t *ts, int s0, int n) {
  return __builtin_amdgcn_make_buffer_rsrc(ts ? const_cast<int32_t *>(ts + s0) : nullptr, 0,
                                           ts ? n * 4 : 0, 0x00020000);
}

__device__ __forceinline__ int32_t load_ts(__amdgpu_buffer_rsrc_t rs, int row, int r0) {
  return __builtin_amdgcn_raw_buffer_load_b32(rs, row * 4, r0 * 4, 0);
}

// Workgroup barrier that orders LDS only: this wave's LDS reads and writes are complete
// (lgkmcnt 0), while its global loads and stores stay in flight (the barrier of
// __syncthreads also waits for every store, which here would hold each wave at every
// tile until its dS stores had reached memory).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt 63 (no wait), expcnt 7 (no wait), lgkmcnt 0
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Registers of one tile of ROWS rows of an fp16 matrix, spread over the workgroup:
// chunk tid + 256 c for c < N.  Each lane's byte offset within the tile is fixed; the
// tile's first row goes in the uniform offset.
template <int DH, int ROWS>
struct TileRegs {
  static constexpr int CHUNKS = ROWS * BwdLayout<DH>::CPR;
  static constexpr int N = (CHUNKS + kThreads - 1) / kThreads;
  u32x4 v[N];

  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int64_t stride, int r0) {
    constexpr int CPR = BwdLayout<DH>::CPR;
    const int soff = (int)((int64_t)r0 * stride * 2);
#pragma unroll
    for (int c = 0; c < N; ++c) {
      const int idx = threadIdx.x + c * kThreads;
      const int r = idx / CPR, ch = idx % CPR;
      v[c] = u32x4{0, 0, 0, 0};
      if (CHUNKS % kThreads == 0 || idx < CHUNKS)
        v[c] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (r * (int)stride + ch * 8) * 2, soff, 0));
    }
  }
  // into a transposed-read copy only
  __device__ __forceinline__ void store_tr(unsigned char *tr_copy) const {
    using L = BwdLayout<DH>;
#pragma unroll
    for (int c = 0; c < N; ++c) {
      const int idx = threadIdx.x + c * kThreads;
      if (CHUNKS % kThreads != 0 && idx >= CHUNKS) break;
      const int r = idx / L::CPR, ch = idx % L::CPR;
      *reinterpret_cast<u32x4 *>(tr_copy + r * L::TRP + ch * 16) = v[c];
    }
  }
  // into a row copy and, with TR, a transposed-read copy too
  template <bool TR>
  __device__ __forceinline__ void store(unsigned char *row_copy, unsigned char *tr_copy) const {
    using L = BwdLayout<DH>;
#pragma unroll
    for (int c = 0; c < N; ++c) {
      const int idx = threadIdx.x + c * kThreads;
      if (CHUNKS % kThreads != 0 && idx >= CHUNKS) break;
      const int r = idx / L::CPR, ch = idx % L::CPR;
      *reinterpret_cast<u32x4 *>(row_copy + r * L::ROWP + ch * 16) = v[c];
      if constexpr (TR) *reinterpret_cast<u32x4 *>(tr_copy + r * L::TRP + ch * 16) = v[c];
    }
  }
};

// Fragment of row (lane % 32) of a row copy for k-step ks: 8 features 16 ks + 8 (lane / 32)
template <int DH>
__device__ __forceinline__ f16x8 row_frag(const unsigned char *row_copy, int lane, int ks) {
  using L = BwdLayout<DH>;
  return as_f16x8(*reinterpret_cast<const u32x4 *>(row_copy + (lane & 31) * L::ROWP +
                                                    (2 * ks + (lane >> 5)) * 16));
}

// Transposed operand for feature tile f and k-step s2 of a 32-row block: rows
// 16 s2 + 8 (e / 4) + 4 (lane / 32) + e % 4 (e = 0..7) of feature 32 f + lane % 32
template <int DH>
__device__ __forceinline__ f16x8 tr_frag(const unsigned char *tr_copy, int lane, int f, int s2) {
  using L = BwdLayout<DH>;
  const int row = 4 * (lane >> 5) + ((lane & 15) >> 2);
  const int col = (32 * f + 16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;
  const u32x2 lo = tr_read(tr_copy + (16 * s2 + row) * L::TRP + col);
  const u32x2 hi = tr_read(tr_copy + (16 * s2 + 8 + row) * L::TRP + col);
  return as_f16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
}

__device__ __forceinline__ f16x8 f16_row_frag(const uint16_t *rowp, bool ok, int lane, int ks) {
  if (!ok) return as_f16x8(u32x4{0, 0, 0, 0});
  return as_f16x8(*reinterpret_cast<const u32x4 *>(rowp + 16 * ks + 8 * (lane >> 5)));
}

// packs accumulator values v[0..7] into the fp16 k-step operand
__device__ __forceinline__ f16x8 pack8(const float *v) {
  return as_f16x8(u32x4{pack_f16(v[0], v[1]), pack_f16(v[2], v[3]), pack_f16(v[4], v[5]),
                        pack_f16(v[6], v[7])});
}

// SiLU(s) and SiLU'(s) = sigma + a (1 - sigma), a = s sigma
__device__ __forceinline__ void silu_and_grad(float s, float &a, float &g) {
  const float sig = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(kNegLog2e * s));
  a = s * sig;
  g = __builtin_fmaf(-a, sig, sig + a);
}

__device__ __forceinline__ float silu_grad(float s) {
  float a, g;
  silu_and_grad(s, a, g);
  return g;
}

struct BiasCtx {
  const float *ptab;
  const float *ttab;
  int pos_buckets, time_buckets;
  bool use_pos, use_time;
};

__device__ __forceinline__ float rab(const BiasCtx &c, int qi, int kj, int32_t qts, int32_t kts) {
  float x = 0.0f;
  if (c.use_pos) x += c.ptab[min(max(qi - kj, 0), c.pos_buckets - 1)];
  if (c.use_time) x += c.ttab[min(time_log2_bucket(qts, kts), c.time_buckets - 1)];
  return x;
}

// Bias class of the block of queries [q_lo, q_lo + 31] x keys [k_lo, k_lo + 31], given
// the (min, max) timestamps of its query and key rows.  CONST: every pair takes lo.
// TWO: a pair takes hi when its gap ts_q - ts_k reaches thr, lo otherwise.  The time
// bucket is at most 32, so thr = 2^(lower bucket + 1) - 1 fits 32 bits whenever TWO is
// chosen (the lower bucket is then below the upper one, at most 31).
struct BlockBias {
  int kind;
  int tb;  // the lower time bucket (CONST: the block's; TWO: hi pairs take tb + 1)
  float lo, hi;
  uint32_t thr;
};

__device__ __forceinline__ BlockBias classify(const BiasCtx &c, int q_lo, int k_lo, int2 tq,
                                              int2 tk) {
  BlockBias r;
  const bool pos_const = !c.use_pos || q_lo - (k_lo + 31) >= c.pos_buckets - 1;
  int tb_lo = 0, tb_hi = 0;
  if (c.use_time) {
    tb_lo = min(time_log2_bucket(tq.x, tk.y), c.time_buckets - 1);
    tb_hi = min(time_log2_bucket(tq.y, tk.x), c.time_buckets - 1);
  }
  r.kind = (!pos_const || tb_hi > tb_lo + 1) ? KIND_GENERAL : (tb_hi == tb_lo ? KIND_CONST : KIND_TWO);
  const float base = c.use_pos ? c.ptab[c.pos_buckets - 1] : 0.0f;
  r.lo = base + (c.use_time ? c.ttab[tb_lo] : 0.0f);
  r.hi = base + (c.use_time ? c.ttab[tb_hi] : 0.0f);
  r.thr = (uint32_t)(((uint64_t)1 << (tb_lo + 1)) - 1);
  r.tb = tb_lo;
  return r;
}

// Scale of the fp16 copy of dO: 2^-e with max |dO| = m 2^e, m in [0.5, 1) (e clamped to
// [-100, 120]); 1 when the maximum is 0 or not finite.  Sets inv to the inverse, 2^e.
__device__ __forceinline__ float d_scale(const uint32_t *d_max, float &inv) {
  const float m = __builtin_bit_cast(float, *d_max);
  if (!(m > 0.0f) || !(m <= 3.402823466e38f)) {
    inv = 1.0f;
    return 1.0f;
  }
  int e;
  (void)frexpf(m, &e);
  e = min(max(e, -100), 120);
  inv = ldexpf(1.0f, e);
  return ldexpf(1.0f, -e);
}

__global__ __launch_bounds__(64) void bwd_clear_kernel(uint32_t *d_max) {
  if (threadIdx.x == 0) *d_max = 0u;
}

// max |d_out| over n4 groups of 4 floats: the magnitude bits (ordered as unsigned
// integers for non-negative floats) reduced per wave, then per workgroup, then one atomic
// per workgroup
__global__ __launch_bounds__(256) void bwd_absmax_kernel(const float *d_out, int64_t n4,
                                                         uint32_t *d_max) {
  __shared__ uint32_t wmax[4];
  uint32_t m = 0u;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    const f32x4 v = reinterpret_cast<const f32x4 *>(d_out)[i];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // copy to a scalar first: a bit cast taken straight from a vector element is
      // miscompiled by this compiler (only element 0 survives)
      const float x = v[j];
      m = max(m, __builtin_bit_cast(uint32_t, x) & 0x7fffffffu);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) atomicMax(d_max, max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3])));
}

__global__ __launch_bounds__(256) void bwd_cast_kernel(const float *d_out, int64_t n4,
                                                       const uint32_t *d_max, uint16_t *d_h) {
  float inv;
  const float sc = d_scale(d_max, inv);
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    const f32x4 v = reinterpret_cast<const f32x4 *>(d_out)[i];
    reinterpret_cast<u32x2 *>(d_h)[i] =
        u32x2{pack_f16(v[0] * sc, v[1] * sc), pack_f16(v[2] * sc, v[3] * sc)};
  }
}

// bf16 dz = acc x inv x SiLU'(z) for one lane's 4 x FT values of a row: features
// f 32 + g 8 + (0..3) from element base (the lane's 4-feature offset already added)
template <int FT>
__device__ __forceinline__ void store_dz(const f32x16 *acc, float inv, const AttnBwdArgs &p,
                                         int64_t base) {
#pragma unroll
  for (int f = 0; f < FT; ++f)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int64_t e = base + f * 32 + g * 8;
      const u32x2 zz = *reinterpret_cast<const u32x2 *>(p.z + e);
      const float z[4] = {f16_lo(zz[0]), f16_hi(zz[0]), f16_lo(zz[1]), f16_hi(zz[1])};
      float r[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) r[j] = acc[f][4 * g + j] * inv * silu_grad(z[j]);
      *reinterpret_cast<u32x2 *>(p.dz + e) = u32x2{pack_bf16(r[0], r[1]), pack_bf16(r[2], r[3])};
    }
}

__device__ __forceinline__ void load_tables(const AttnBwdArgs &p, int h, float *ptab, float *ttab,
                                            BiasCtx &bc) {
  const int rrow = p.rab_per_head ? h : 0;
  bc = BiasCtx{ptab, ttab, p.pos_buckets, p.time_buckets, p.rab_pos != nullptr,
               p.rab_time != nullptr && p.ts != nullptr};
  if (bc.use_pos)
    for (int i = threadIdx.x; i < p.pos_buckets; i += kThreads) ptab[i] = p.rab_pos[rrow * p.pos_buckets + i];
  if (bc.use_time)
    for (int i = threadIdx.x; i < p.time_buckets; i += kThreads) ttab[i] = p.rab_time[rrow * p.time_buckets + i];
}

// Sums of dS per bias bucket for one wave: the gradients of the bias tables, every
// allowed pair's dS going to its position and time bucket.  Blocks whose position bucket
// is P - 1 throughout add their dS to a per-lane sum pos_run; CONST blocks add theirs to
// t_run for the current time bucket t_run_b, which changes only a few times along a
// wave's blocks, and TWO blocks reduce their two time sums at once.  GENERAL blocks add
// each pair to the wave's bins with LDS atomics: the time bucket is mostly shared by a
// wave's lanes, so each lane adds into its own copy of the time bins.
struct RabAcc {
  float *wpos, *wtime, *ltime;
  int PB, TB, lane;
  bool use_pos, use_time;
  float pos_run, t_run;
  int t_run_b;

  __device__ __forceinline__ void init(float *pos_bins, float *time_bins, int lane_,
                                       const BiasCtx &bc) {
    wpos = pos_bins;
    wtime = time_bins;
    ltime = time_bins + (lane_ % kTimeReps) * kTimeRepPitch;
    PB = bc.pos_buckets;
    TB = bc.time_buckets;
    lane = lane_;
    use_pos = bc.use_pos;
    use_time = bc.use_time;
    pos_run = t_run = 0.0f;
    t_run_b = 0;
    for (int i = lane; i < PB; i += 64) wpos[i] = 0.0f;
    for (int i = lane; i < kTimeReps * kTimeRepPitch; i += 64) wtime[i] = 0.0f;
  }
  __device__ __forceinline__ static float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
  }
  // the lane's value into its own copy of the time bins (lane % kTimeReps): one LDS atomic,
  // no cross-lane sum (six dependent shuffles per call cost more than the whole block's
  // bin update); the copies are summed once, in rab_write
  __device__ __forceinline__ void time_add(float v, int b) { atomicAdd(&ltime[b], v); }
  // One 32 x 32 block: the lane's query qi (q_ok) and its 16 values ds[i] for the keys
  // kb + 8 (i / 4) + 4 half + i % 4, whose timestamps are kts[8 (i / 4) + i % 4].
  __device__ __forceinline__ void block(const BlockBias &bb, const float *ds, const int32_t *kts,
                                        int32_t klim, int kb, int qbase, int qi, bool q_ok,
                                        int half, int32_t qts) {
    if (bb.kind == KIND_CONST) {
      float sum = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) sum += ds[i];
      add_const(bb, sum);
    } else if (bb.kind == KIND_TWO) {
      float shi = 0.0f, slo = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const bool hi = kts[8 * (i >> 2) + (i & 3)] < klim;
        shi += hi ? ds[i] : 0.0f;
        slo += hi ? 0.0f : ds[i];
      }
      pos_run += shi + slo;
      time_add(slo, bb.tb);
      time_add(shi, bb.tb + 1);
    } else {
      const bool pos_each = use_pos && qbase - (kb + 31) < PB - 1;  // near the diagonal
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kj = kb + 8 * (i >> 2) + 4 * half + (i & 3);
        if (q_ok && kj <= qi) {
          if (pos_each) atomicAdd(&wpos[min(qi - kj, PB - 1)], ds[i]);
          else pos_run += ds[i];
          if (use_time)
            atomicAdd(&ltime[min(time_log2_bucket(qts, kts[8 * (i >> 2) + (i & 3)]), TB - 1)], ds[i]);
        }
      }
    }
  }
  // a CONST block, given the sum of the lane's 16 values
  __device__ __forceinline__ void add_const(const BlockBias &bb, float sum) {
    pos_run += sum;
    if (use_time) {
      if (bb.tb != t_run_b) {
        time_add(t_run, t_run_b);
        t_run = 0.0f;
        t_run_b = bb.tb;
      }
      t_run += sum;
    }
  }
  __device__ __forceinline__ void flush() {
    if (use_time) time_add(t_run, t_run_b);
    if (use_pos) {
      const float v = wave_sum(pos_run);
      if (lane == 0) wpos[PB - 1] += v;
    }
  }
};

// The workgroup's bins (after a barrier), summed in a fixed order, into its slot of the
// per-work-item partials.
__device__ __forceinline__ void rab_write(const AttnBwdArgs &p, const float (*rpos)[kMaxPos],
                                          const float (*rtime)[kTimeReps][kTimeRepPitch], int h,
                                          int item) {
  const int PB = p.pos_buckets;
  const int nb = PB + p.time_buckets;
  float *dst = p.rab_part + ((int64_t)h * p.rab_cap + item) * nb;
  for (int i = threadIdx.x; i < nb; i += kThreads) {
    float t = 0.0f;
    if (i < PB) {
      for (int w = 0; w < kWaves; ++w) t += rpos[w][i];
    } else {
      for (int w = 0; w < kWaves; ++w)
        for (int r = 0; r < kTimeReps; ++r) t += rtime[w][r][i - PB];
    }
    dst[i] = t;
  }
}

// -------------------------------------------------------------------------------------
// dQ: queries owned, keys streamed
// -------------------------------------------------------------------------------------
template <int DH>
__global__ __launch_bounds__(kThreads, 2) void attn_bwd_dq_kernel(AttnBwdArgs p) {
  using L = BwdLayout<DH>;
  constexpr int KS = L::KS, FT = L::FT;
  constexpr int TK = dq_keys<DH>();
  __shared__ __attribute__((aligned(16))) unsigned char k_row[TK * L::ROWP];
  __shared__ __attribute__((aligned(16))) unsigned char k_tr[TK * L::TRP];
  __shared__ __attribute__((aligned(16))) unsigned char v_row[TK * L::ROWP];
  __shared__ int32_t k_ts[TK];
  __shared__ float ptab[kMaxPos], ttab[kMaxTime];
  // per-wave sums of dS per bucket: position bins, and time bins in kTimeReps copies
  // (lane l adds into copy l % kTimeReps, whose bins sit one bank apart)
  __shared__ float rpos[kWaves][kMaxPos];
  __shared__ float rtime[kWaves][kTimeReps][kTimeRepPitch];

  const int item = blockIdx.x;
  if (item >= ld_const(p.n_work)) return;
  const int h = blockIdx.y;
  const int b = ld_const(p.work + 2 * item), qt = ld_const(p.work + 2 * item + 1);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar row ranges
  const int lrow = lane & 31, half = lane >> 5;
  const int s0 = ld_const(p.offsets + b), n = ld_const(p.offsets + b + 1) - s0;
  BiasCtx bc;
  load_tables(p, h, ptab, ttab, bc);

  const int q0 = qt * kOwnRows;
  const int qbase = q0 + wave * 32;  // this wave's 32 queries
  const bool wave_rows = qbase < n;
  const int qi = qbase + lrow;
  const bool q_ok = qi < n;
  const int32_t qts = bc.use_time ? p.ts[s0 + (q_ok ? qi : 0)] : 0;
  const int2 tq = (bc.use_time && wave_rows) ? ld_stat(p.stat + s0 + qbase) : int2{0, 0};
  f16x8 qf[KS], dof[KS];
  {
    const uint16_t *qr = p.q + (int64_t)(s0 + qi) * p.stride + h * DH;
    const uint16_t *dr = p.d_h + (int64_t)(s0 + qi) * p.d_stride + h * DH;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks] = f16_row_frag(qr, q_ok, lane, ks);
      dof[ks] = f16_row_frag(dr, q_ok, lane, ks);
    }
  }
  f32x16 acc[FT];
#pragma unroll
  for (int f = 0; f < FT; ++f) acc[f] = f32x16{};

  const bool want_rab = p.rab_part != nullptr && (bc.use_pos || bc.use_time);
  RabAcc ra;
  if (want_rab) ra.init(rpos[wave], &rtime[wave][0][0], lane, bc);

  const __amdgpu_buffer_rsrc_t krs = rows_rsrc(p.k + (int64_t)s0 * p.stride + h * DH, p.stride, n, DH);
  const __amdgpu_buffer_rsrc_t vrs = rows_rsrc(p.v + (int64_t)s0 * p.stride + h * DH, p.stride, n, DH);
  const int k_end = min(n, q0 + kOwnRows);  // keys j <= i < q0 + 128
  const int n_tiles = (k_end + TK - 1) / TK;
  const __amdgpu_buffer_rsrc_t trs = ts_rsrc(bc.use_time ? p.ts : nullptr, s0, n);
  TileRegs<DH, TK> rk, rv;
  int32_t rts = 0;
  auto prefetch = [&](int j0) __attribute__((always_inline)) {
    rk.load(krs, p.stride, j0);
    rv.load(vrs, p.stride, j0);
    if (tid < TK) rts = load_ts(trs, tid, j0);
  };
  prefetch(0);
  for (int t = 0; t < n_tiles; ++t) {
    const int j0 = t * TK;
    __syncthreads();  // the previous tile is no longer read (and the tables are written)
    rk.template store<true>(k_row, k_tr);
    rv.template store<false>(v_row, nullptr);
    if (tid < TK) k_ts[tid] = rts;
    __syncthreads();
    if (t + 1 < n_tiles) prefetch(j0 + TK);
#pragma unroll
    for (int blk = 0; blk < TK / 32; ++blk) {
      const int kb = j0 + 32 * blk;
      if (!wave_rows || kb > qbase + 31 || kb >= n) continue;  // uniform per wave
      const unsigned char *kr = k_row + blk * 32 * L::ROWP;
      const unsigned char *ktr = k_tr + blk * 32 * L::TRP;
      const unsigned char *vr = v_row + blk * 32 * L::ROWP;
      const int32_t *kts = k_ts + blk * 32 + 4 * half;
      const int2 tk = bc.use_time ? ld_stat(p.stat + s0 + kb) : int2{0, 0};
      const BlockBias bb = classify(bc, qbase, kb, tq, tk);
      // S^T with its bias, dA^T; lane: query lrow, keys 8 (i / 4) + 4 half + i % 4
      f32x16 s, da = f32x16{};
      const int64_t lim = (int64_t)qts - (int64_t)bb.thr + 1;  // TWO: hi when ts_k < lim
      const int32_t klim = (int32_t)(lim < (int64_t)INT32_MIN ? (int64_t)INT32_MIN : lim);
      if (bb.kind == KIND_CONST) {
#pragma unroll
        for (int i = 0; i < 16; ++i) s[i] = bb.lo;
      } else if (bb.kind == KIND_TWO) {
#pragma unroll
        for (int i = 0; i < 16; ++i) s[i] = kts[8 * (i >> 2) + (i & 3)] < klim ? bb.hi : bb.lo;
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          s[i] = rab(bc, qi, kb + 8 * (i >> 2) + 4 * half + (i & 3), qts, kts[8 * (i >> 2) + (i & 3)]);
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s = mfma32_f16(row_frag<DH>(kr, lane, ks), qf[ks], s);
        da = mfma32_f16(row_frag<DH>(vr, lane, ks), dof[ks], da);
      }
      float ds[16];
      if (kb + 31 > qbase) {  // straddles the diagonal: keys after the query are masked
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kj = kb + 8 * (i >> 2) + 4 * half + (i & 3);
          ds[i] = kj <= qi ? da[i] * silu_grad(s[i]) : 0.0f;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) ds[i] = da[i] * silu_grad(s[i]);
      }
      if (want_rab) ra.block(bb, ds, kts, klim, kb, qbase, qi, q_ok, half, qts);
      // dQ^T += K^T dS^T over the block's 32 keys
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const f16x8 bop = pack8(ds + 8 * s2);
#pragma unroll
        for (int f = 0; f < FT; ++f) acc[f] = mfma32_f16(tr_frag<DH>(ktr, lane, f, s2), bop, acc[f]);
      }
    }
  }
  if (want_rab) {  // flush the runs, then the workgroup's bins in a fixed order
    ra.flush();
    __syncthreads();
    rab_write(p, rpos, rtime, h, item);
  }
  if (q_ok) {
    float inv;
    (void)d_scale(p.d_max, inv);
    if (p.dz != nullptr) {
      store_dz<FT>(acc, inv, p, (int64_t)(s0 + qi) * p.z_stride + p.zq_off + h * DH + half * 4);
    } else {
      float *orow = p.dq + (int64_t)(s0 + qi) * p.g_stride + h * DH + half * 4;
#pragma unroll
      for (int f = 0; f < FT; ++f)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<f32x4 *>(orow + f * 32 + g * 8) =
              f32x4{acc[f][4 * g] * inv, acc[f][4 * g + 1] * inv, acc[f][4 * g + 2] * inv,
                    acc[f][4 * g + 3] * inv};
    }
  }
}

// -------------------------------------------------------------------------------------
// dQ from the stored dS
// -------------------------------------------------------------------------------------
// First block of each sequence's causal triangle of 32 x 32 blocks: tri[b] = the sum over
// b' < b of nb' (nb' + 1) / 2, nb' = ceil(n_b' / 32); tri[B] = the total.  One workgroup:
// per-thread runs of sequences, then an exclusive scan of the runs.
__global__ __launch_bounds__(1024) void tri_base_kernel(const int32_t *offsets, int B, int64_t *tri) {
  __shared__ int64_t part[1024];
  const int t = threadIdx.x, per = (B + 1023) / 1024;
  const int b0 = min(B, t * per), b1 = min(B, b0 + per);
  auto blocks = [&](int b) {
    const int64_t nb = (offsets[b + 1] - offsets[b] + 31) / 32;
    return nb * (nb + 1) / 2;
  };
  int64_t sum = 0;
  for (int b = b0; b < b1; ++b) sum += blocks(b);
  part[t] = sum;
  __syncthreads();
  if (t == 0) {
    int64_t run = 0;
    for (int i = 0; i < 1024; ++i) {
      const int64_t v = part[i];
      part[i] = run;
      run += v;
    }
    tri[B] = run;
  }
  __syncthreads();
  int64_t run = part[t];
  for (int b = b0; b < b1; ++b) {
    tri[b] = run;
    run += blocks(b);
  }
}

// A stored block in LDS: its two 1 KB halves (the dK/dV kernel's lanes 0..63, 16 bytes
// each) at kDsHalf bytes apart, lanes 32..63 of a half 64 bytes further on, so that the
// transposing reads below fall on distinct banks: the reads of lanes 0..15 cover banks
// 0..31 of one half, those of lanes 16..31 the same pattern in the other half, which
// kDsHalf (288 banks, 32 mod 64) moves onto banks 32..63.
constexpr int kDsHalf = 1152;
constexpr int kDsBlock = 2 * kDsHalf;
__device__ __forceinline__ int ds_lds_offset(int piece) {  // 16-byte piece of the 2 KB block
  const int half = piece >> 6, L = piece & 63;
  return half * kDsHalf + L * 16 + (L >= 32 ? 64 : 0);
}

// Transposed operand of a stored block for k-step s2: keys 16 s2 + 8 (e / 4) +
// 4 (lane / 32) + e % 4 (e = 0..7) of query lane % 32, the key order of tr_frag.  The
// transposing read takes, per 16-lane group, 4 keys x 4 groups of 4 queries; queries
// 4 m .. 4 m + 3 of key k sit in the dK/dV lane k + 32 (m % 2) of half m / 4, at values
// 4 ((m / 2) % 2) .. + 3.
__device__ __forceinline__ f16x8 ds_frag(const unsigned char *blk, int lane, int s2) {
  const int g = lane >> 4, c = lane & 3, jr = (lane & 15) >> 2;
  const int base = (g & 1) * kDsHalf + 64 * (c & 1) + 8 * (c >> 1) + 32 * (c & 1) * 16;
  const int k = 16 * s2 + 4 * (lane >> 5) + jr;
  const u32x2 lo = tr_read(blk + base + k * 16);
  const u32x2 hi = tr_read(blk + base + (k + 8) * 16);
  return as_f16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
}

// A workgroup owns 128 queries and streams 64-key tiles: the K rows (transposed-read
// copy) and, per wave, the two stored dS blocks of its 32 queries.  Per block
// dQ^T += K^T dS^T (8 MFMAs at DH = 128), both operands through the transposing read; no
// scores, dA or SiLU' are formed again.  The bias-table sums read the same dS values.
template <int DH>
__global__ __launch_bounds__(kThreads, 2) void attn_bwd_dq_ds_kernel(AttnBwdArgs p) {
  using L = BwdLayout<DH>;
  constexpr int FT = L::FT;
  constexpr int TK = 64;
  __shared__ __attribute__((aligned(16))) unsigned char k_tr[TK * L::TRP];
  __shared__ __attribute__((aligned(16))) unsigned char ds_l[kWaves][TK / 32][kDsBlock];
  __shared__ int32_t k_ts[TK];
  __shared__ float ptab[kMaxPos], ttab[kMaxTime];
  __shared__ float rpos[kWaves][kMaxPos];
  __shared__ float rtime[kWaves][kTimeReps][kTimeRepPitch];

  const int item = blockIdx.x;
  if (item >= ld_const(p.n_work)) return;
  const int h = blockIdx.y;
  const int b = ld_const(p.work + 2 * item), qt = ld_const(p.work + 2 * item + 1);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lrow = lane & 31, half = lane >> 5;
  const int s0 = ld_const(p.offsets + b), n = ld_const(p.offsets + b + 1) - s0;
  BiasCtx bc;
  load_tables(p, h, ptab, ttab, bc);

  const int q0 = qt * kOwnRows;
  const int qbase = q0 + wave * 32;
  const bool wave_rows = qbase < n;
  const int qi = qbase + lrow;
  const bool q_ok = qi < n;
  const bool want_rab = p.rab_part != nullptr && (bc.use_pos || bc.use_time);
  const int32_t qts = (want_rab && bc.use_time) ? p.ts[s0 + (q_ok ? qi : 0)] : 0;
  const int2 tq = (want_rab && bc.use_time && wave_rows) ? ld_stat(p.stat + s0 + qbase) : int2{0, 0};
  RabAcc ra;
  if (want_rab) ra.init(rpos[wave], &rtime[wave][0][0], lane, bc);
  f32x16 acc[FT];
#pragma unroll
  for (int f = 0; f < FT; ++f) acc[f] = f32x16{};

  const __amdgpu_buffer_rsrc_t krs = rows_rsrc(p.k + (int64_t)s0 * p.stride + h * DH, p.stride, n, DH);
  const __amdgpu_buffer_rsrc_t trs = ts_rsrc(bc.use_time ? p.ts : nullptr, s0, n);
  const int k_end = min(n, q0 + kOwnRows);
  const int n_tiles = (k_end + TK - 1) / TK;
  const int64_t head0 = (int64_t)h * p.ds_head_blocks + ld_const(p.tri_base + b);
  const int nq_blocks = (n + 31) / 32;
  // the tile's stored blocks: 16-byte piece c of the 16 KB, c = tid + 256 i: wave c / 256,
  // block (c / 128) % 2 of the tile, piece c % 128; absent blocks (after the diagonal or
  // past the sequence) read as zero
  TileRegs<DH, TK> rk;
  u32x4 rds[4];
  int32_t rts = 0;
  auto prefetch = [&](int j0) __attribute__((always_inline)) {
    rk.load(krs, p.stride, j0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;
      const int qb = q0 / 32 + (c >> 8), kb = j0 / 32 + ((c >> 7) & 1);
      rds[i] = u32x4{0, 0, 0, 0};
      if (qb < nq_blocks && kb <= qb)
        rds[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(
            p.ds_buf + (head0 + (int64_t)qb * (qb + 1) / 2 + kb) * 1024 + (c & 127) * 8));
    }
    if (tid < TK) rts = load_ts(trs, tid, j0);
  };
  prefetch(0);
  for (int t = 0; t < n_tiles; ++t) {
    const int j0 = t * TK;
    __syncthreads();  // the previous tile is no longer read (and the tables are written)
    rk.store_tr(k_tr);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;
      *reinterpret_cast<u32x4 *>(&ds_l[c >> 8][(c >> 7) & 1][ds_lds_offset(c & 127)]) = rds[i];
    }
    if (tid < TK) k_ts[tid] = rts;
    __syncthreads();
    if (t + 1 < n_tiles) prefetch(j0 + TK);
    int2 tks[TK / 32];  // the blocks' key timestamp ranges, loaded ahead of their use
#pragma unroll
    for (int blk = 0; blk < TK / 32; ++blk)
      tks[blk] = (want_rab && bc.use_time && j0 + 32 * blk < n) ? ld_stat(p.stat + s0 + j0 + 32 * blk)
                                                                : int2{0, 0};
#pragma unroll
    for (int blk = 0; blk < TK / 32; ++blk) {
      const int kb = j0 + 32 * blk;
      if (!wave_rows || kb > qbase + 31 || kb >= n) continue;  // uniform per wave
      const unsigned char *ktr = k_tr + blk * 32 * L::TRP;
      const f16x8 d0 = ds_frag(ds_l[wave][blk], lane, 0), d1 = ds_frag(ds_l[wave][blk], lane, 1);
#pragma unroll
      for (int f = 0; f < FT; ++f) {
        acc[f] = mfma32_f16(tr_frag<DH>(ktr, lane, f, 0), d0, acc[f]);
        acc[f] = mfma32_f16(tr_frag<DH>(ktr, lane, f, 1), d1, acc[f]);
      }
      if (want_rab) {
        const BlockBias bb = classify(bc, qbase, kb, tq, tks[blk]);
        if (bb.kind == KIND_CONST) {  // the lane's sum by packed dot products with ones
          typedef _Float16 h2 __attribute__((ext_vector_type(2)));
          const h2 one = {(_Float16)1.0f, (_Float16)1.0f};
          float sum = 0.0f;
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            sum = __builtin_amdgcn_fdot2(h2{d0[e], d0[e + 1]}, one, sum, false);
            sum = __builtin_amdgcn_fdot2(h2{d1[e], d1[e + 1]}, one, sum, false);
          }
          ra.add_const(bb, sum);
        } else {
          float ds[16];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            ds[e] = (float)d0[e];
            ds[8 + e] = (float)d1[e];
          }
          const int64_t lim = (int64_t)qts - (int64_t)bb.thr + 1;  // TWO: hi when ts_k < lim
          const int32_t klim = (int32_t)(lim < (int64_t)INT32_MIN ? (int64_t)INT32_MIN : lim);
          ra.block(bb, ds, k_ts + blk * 32 + 4 * half, klim, kb, qbase, qi, q_ok, half, qts);
        }
      }
    }
  }
  if (want_rab) {
    ra.flush();
    __syncthreads();
    rab_write(p, rpos, rtime, h, item);
  }
  if (q_ok) {
    float inv;
    (void)d_scale(p.d_max, inv);
    if (p.dz != nullptr) {
      store_dz<FT>(acc, inv, p, (int64_t)(s0 + qi) * p.z_stride + p.zq_off + h * DH + half * 4);
    } else {
      float *orow = p.dq + (int64_t)(s0 + qi) * p.g_stride + h * DH + half * 4;
#pragma unroll
      for (int f = 0; f < FT; ++f)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<f32x4 *>(orow + f * 32 + g * 8) =
              f32x4{acc[f][4 * g] * inv, acc[f][4 * g + 1] * inv, acc[f][4 * g + 2] * inv,
                    acc[f][4 * g + 3] * inv};
    }
  }
}

// -------------------------------------------------------------------------------------
// dK, dV: keys owned, queries streamed
// -------------------------------------------------------------------------------------
// Two workgroups per CU at every head size: at DH = 128 the dK and dV accumulators (128
// registers), the K fragments (32) and one half of A and dS at a time fit 256 registers.
template <int DH>
__global__ __launch_bounds__(kThreads, 2) void attn_bwd_dkv_kernel(AttnBwdArgs p) {
  using L = BwdLayout<DH>;
  constexpr int KS = L::KS, FT = L::FT;
  constexpr int TQ = kDkvQueries;
  __shared__ __attribute__((aligned(16))) unsigned char q_row[TQ * L::ROWP];
  __shared__ __attribute__((aligned(16))) unsigned char q_tr[TQ * L::TRP];
  __shared__ __attribute__((aligned(16))) unsigned char d_row[TQ * L::ROWP];
  __shared__ __attribute__((aligned(16))) unsigned char d_tr[TQ * L::TRP];
  __shared__ __attribute__((aligned(16))) unsigned char v_own[kOwnRows * L::ROWP];
  __shared__ int32_t q_ts[TQ];
  __shared__ float ptab[kMaxPos], ttab[kMaxTime];

  const int item = blockIdx.x;
  if (item >= ld_const(p.n_work)) return;
  const int h = blockIdx.y;
  const int b = ld_const(p.work + 2 * item);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar row ranges
  const int lrow = lane & 31, half = lane >> 5;
  const int s0 = ld_const(p.offsets + b), n = ld_const(p.offsets + b + 1) - s0;
  // the list is ordered for the query tiles (tile t visits t + 1 key tiles); key tile
  // nt - 1 - t visits as many query tiles, so the reversal keeps the longest items first
  const int kt = (n + kOwnRows - 1) / kOwnRows - 1 - ld_const(p.work + 2 * item + 1);
  const int64_t tri0 = p.ds_buf != nullptr ? ld_const(p.tri_base + b) : 0;
  BiasCtx bc;
  load_tables(p, h, ptab, ttab, bc);

  const int k0 = kt * kOwnRows;
  const int kbase = k0 + wave * 32;  // this wave's 32 keys
  const bool wave_rows = kbase < n;
  const int kj = kbase + lrow;
  const bool k_ok = kj < n;
  const int32_t kts = bc.use_time ? p.ts[s0 + (k_ok ? kj : 0)] : 0;
  const int2 tk = (bc.use_time && wave_rows) ? ld_stat(p.stat + s0 + kbase) : int2{0, 0};
  f16x8 kf[KS];
  {
    const uint16_t *kr = p.k + (int64_t)(s0 + kj) * p.stride + h * DH;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kf[ks] = f16_row_frag(kr, k_ok, lane, ks);
  }
  {  // the workgroup's V rows, read as B operands of dA = dO V^T
    TileRegs<DH, kOwnRows> rv;
    rv.load(rows_rsrc(p.v + (int64_t)s0 * p.stride + h * DH, p.stride, n, DH), p.stride, k0);
    rv.template store<false>(v_own, nullptr);
  }
  const unsigned char *vw = v_own + wave * 32 * L::ROWP;
  f32x16 dk_acc[FT], dv_acc[FT];
#pragma unroll
  for (int f = 0; f < FT; ++f) dk_acc[f] = dv_acc[f] = f32x16{};

  const __amdgpu_buffer_rsrc_t qrs = rows_rsrc(p.q + (int64_t)s0 * p.stride + h * DH, p.stride, n, DH);
  const __amdgpu_buffer_rsrc_t drs =
      rows_rsrc(p.d_h + (int64_t)s0 * p.d_stride + h * DH, p.d_stride, n, DH);
  const int n_tiles = (n - k0 + TQ - 1) / TQ;  // queries i >= k0 see these keys
  const __amdgpu_buffer_rsrc_t trs = ts_rsrc(bc.use_time ? p.ts : nullptr, s0, n);
  TileRegs<DH, TQ> rq, rd;
  int32_t rts = 0;
  // Every tile's loads are issued by every thread on every path (past the sequence end
  // they read zero), and with dS kept every path then issues two stores, so the wait for a
  // tile's loads has the same form on every path and leaves the stores in flight.
  auto prefetch = [&](int i0) __attribute__((always_inline)) {
    rq.load(qrs, p.stride, i0);
    rd.load(drs, p.d_stride, i0);
    rts = load_ts(trs, tid, i0);
  };
  auto dump_stores = [&]() __attribute__((always_inline)) {
    __builtin_nontemporal_store(u32x4{0, 0, 0, 0}, reinterpret_cast<u32x4 *>(p.ds_dump + 8 * lane));
    __builtin_nontemporal_store(u32x4{0, 0, 0, 0}, reinterpret_cast<u32x4 *>(p.ds_dump + 512 + 8 * lane));
  };
  prefetch(k0);
  if (p.ds_buf != nullptr) dump_stores();
  for (int t = 0; t < n_tiles; ++t) {
    const int i0 = k0 + t * TQ;
    lds_barrier();  // the previous tile is no longer read (tables and V rows written)
    rq.template store<true>(q_row, q_tr);
    rd.template store<true>(d_row, d_tr);
    if (tid < TQ) q_ts[tid] = rts;
    lds_barrier();
    prefetch(i0 + TQ);
    if (!wave_rows || i0 + 31 < kbase) {  // every query precedes this wave's keys
      // (loads and stores share one in-order counter: a skipped block writes zeros to a
      // slot that nothing reads, so that this path too issues two stores)
      if (p.ds_buf != nullptr) dump_stores();
      continue;
    }
    const int2 tq = bc.use_time ? ld_stat(p.stat + s0 + i0) : int2{0, 0};
    const BlockBias bb = classify(bc, i0, kbase, tq, tk);
    const int32_t *qtsp = q_ts + 4 * half;
    // S and dA; lane: key lrow, queries 8 (e / 4) + 4 half + e % 4 of the tile
    f32x16 s, da = f32x16{};
    if (bb.kind == KIND_CONST) {
#pragma unroll
      for (int e = 0; e < 16; ++e) s[e] = bb.lo;
    } else if (bb.kind == KIND_TWO) {
      // hi when ts_q - ts_k >= thr, i.e. ts_q > ts_k + thr - 1 (never past INT32_MAX)
      const int64_t gt = (int64_t)kts + (int64_t)bb.thr - 1;
      const int32_t qgt = (int32_t)(gt > (int64_t)INT32_MAX ? (int64_t)INT32_MAX : gt);
#pragma unroll
      for (int e = 0; e < 16; ++e) s[e] = qtsp[8 * (e >> 2) + (e & 3)] > qgt ? bb.hi : bb.lo;
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e)
        s[e] = rab(bc, i0 + 8 * (e >> 2) + 4 * half + (e & 3), kj, qtsp[8 * (e >> 2) + (e & 3)], kts);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s = mfma32_f16(row_frag<DH>(q_row, lane, ks), kf[ks], s);
      da = mfma32_f16(row_frag<DH>(d_row, lane, ks), row_frag<DH>(vw, lane, ks), da);
    }
    // A and dS, then dV^T += dO^T A and dK^T += Q^T dS, over the tile's queries in two
    // halves of 16 (8 values per lane each), so that only one half is live in registers
    const bool diag = i0 < kbase + 31;  // straddles the diagonal: earlier queries masked
    uint16_t *ds_blk = nullptr;  // the stored block (query block i0 / 32, this wave's keys)
    if (p.ds_buf != nullptr) {
      const int qb = i0 / 32, kbb = kbase / 32;
      ds_blk = p.ds_buf + ((int64_t)h * p.ds_head_blocks + tri0 + (int64_t)qb * (qb + 1) / 2 + kbb) * 1024;
    }
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      float a[8], ds[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int e = 8 * s2 + j;
        float av, g;
        silu_and_grad(s[e], av, g);
        a[j] = av;
        ds[j] = da[e] * g;
        if (diag) {
          const bool ok = kj <= i0 + 8 * (e >> 2) + 4 * half + (e & 3);
          a[j] = ok ? a[j] : 0.0f;
          ds[j] = ok ? ds[j] : 0.0f;
        }
      }
      const f16x8 aop = pack8(a), dop = pack8(ds);
      if (ds_blk != nullptr)  // the lane's 8 values of this half: 1 KB per wave, contiguous;
        // streamed past the caches, which hold the Q and dO tiles that other workgroups reuse
        __builtin_nontemporal_store(__builtin_bit_cast(u32x4, dop),
                                    reinterpret_cast<u32x4 *>(ds_blk + 512 * s2 + 8 * lane));
#pragma unroll
      for (int f = 0; f < FT; ++f) {
        dv_acc[f] = mfma32_f16(tr_frag<DH>(d_tr, lane, f, s2), aop, dv_acc[f]);
        dk_acc[f] = mfma32_f16(tr_frag<DH>(q_tr, lane, f, s2), dop, dk_acc[f]);
      }
    }
  }
  if (k_ok && p.dz != nullptr) {
    float inv;
    (void)d_scale(p.d_max, inv);
    const int64_t rb = (int64_t)(s0 + kj) * p.z_stride + h * DH + half * 4;
    store_dz<FT>(dk_acc, inv, p, rb + p.zk_off);
    store_dz<FT>(dv_acc, inv, p, rb + p.zv_off);
  } else if (k_ok) {
    float inv;
    (void)d_scale(p.d_max, inv);
    float *kr = p.dk + (int64_t)(s0 + kj) * p.g_stride + h * DH + half * 4;
    float *vr = p.dv + (int64_t)(s0 + kj) * p.g_stride + h * DH + half * 4;
#pragma unroll
    for (int f = 0; f < FT; ++f)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        *reinterpret_cast<f32x4 *>(kr + f * 32 + g * 8) =
            f32x4{dk_acc[f][4 * g] * inv, dk_acc[f][4 * g + 1] * inv, dk_acc[f][4 * g + 2] * inv,
                  dk_acc[f][4 * g + 3] * inv};
        *reinterpret_cast<f32x4 *>(vr + f * 32 + g * 8) =
            f32x4{dv_acc[f][4 * g] * inv, dv_acc[f][4 * g + 1] * inv, dv_acc[f][4 * g + 2] * inv,
                  dv_acc[f][4 * g + 3] * inv};
      }
  }
}

// d rab[row][bin] = 2^e x the sum over the heads of the row (all heads when the tables
// are shared) and the work items of the dQ kernel's per-item bins.  One workgroup per
// (row, bin): thread t sums every 256th (head, item) entry from t, then the 256 partial
// sums are combined in a fixed tree order, so the result does not depend on scheduling.
__global__ __launch_bounds__(256) void rab_reduce_kernel(AttnBwdArgs p, float *d_pos, float *d_time) {
  __shared__ float wsum[kWaves];
  const int nb = p.pos_buckets + p.time_buckets;
  const int row = blockIdx.x / nb, bin = blockIdx.x % nb;
  const int items = ld_const(p.n_work);
  const int h0 = p.rab_per_head ? row : 0, nh = p.rab_per_head ? 1 : p.num_heads;
  float s = 0.0f;
  for (int idx = threadIdx.x; idx < nh * items; idx += 256) {
    const int h = h0 + idx / items, it = idx % items;
    s += p.rab_part[((int64_t)h * p.rab_cap + it) * nb + bin];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x != 0) return;
  float inv;
  (void)d_scale(p.d_max, inv);
  const float t = ((wsum[0] + wsum[1]) + (wsum[2] + wsum[3])) * inv;
  if (bin < p.pos_buckets) {
    if (d_pos) d_pos[row * p.pos_buckets + bin] = t;
  } else if (d_time) {
    d_time[row * p.time_buckets + bin - p.pos_buckets] = t;
  }
}

template <int DH>
hipError_t launch_bwd_dh(const AttnBwdArgs &a, int64_t cap, hipStream_t stream) {
  const dim3 grid((unsigned)cap, (unsigned)a.num_heads);
  if (a.ds_buf != nullptr) {  // dK/dV store dS, then dQ reads it
    tri_base_kernel<<<1, 1024, 0, stream>>>(a.offsets, a.batch, a.tri_base);
    attn_bwd_dkv_kernel<DH><<<grid, dim3(kThreads), 0, stream>>>(a);
    attn_bwd_dq_ds_kernel<DH><<<grid, dim3(kThreads), 0, stream>>>(a);
    return hipGetLastError();
  }
  attn_bwd_dq_kernel<DH><<<grid, dim3(kThreads), 0, stream>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  attn_bwd_dkv_kernel<DH><<<grid, dim3(kThreads), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention_bwd(const AttnBwdArgs &a, int dh, int64_t cap, int64_t total_rows,
                                hipStream_t stream) {
  if (cap <= 0 || a.num_heads <= 0 || total_rows <= 0) return hipSuccess;
  if (dh != 32 && dh != 64 && dh != 128) return hipErrorInvalidValue;
  // the fp16 copy of dO; d_stride = H dh is a multiple of 32, so rows are whole f32x4s
  const int64_t n4 = total_rows * a.d_stride / 4;
  const int blocks = (int)((n4 + 255) / 256 < 1024 ? (n4 + 255) / 256 : 1024);
  bwd_clear_kernel<<<1, 64, 0, stream>>>(a.d_max);
  bwd_absmax_kernel<<<blocks, 256, 0, stream>>>(a.d_out, n4, a.d_max);
  bwd_cast_kernel<<<blocks, 256, 0, stream>>>(a.d_out, n4, a.d_max, a.d_h);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch (dh) {
    case 32: e = launch_bwd_dh<32>(a, cap, stream); break;
    case 64: e = launch_bwd_dh<64>(a, cap, stream); break;
    default: e = launch_bwd_dh<128>(a, cap, stream); break;
  }
  if (e != hipSuccess || a.rab_part == nullptr) return e;
  const int rows = a.rab_per_head ? a.num_heads : 1;
  rab_reduce_kernel<<<rows * (a.pos_buckets + a.time_buckets), 256, 0, stream>>>(a, a.d_rab_pos,
                                                                                 a.d_rab_time);
  return hipGetLastError();
}

}  // namespace hstu
