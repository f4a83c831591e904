// Gradients of the jagged pointwise attention (equation 2 of the layer, "Actions Speak
// Louder than Words" as retold on chenhuiyu.github.io, section "HSTU Layer 到底改了什么"),
// causal mask, no prefix.  Per sequence and head, with S = Q K^T + rab^{p,t},
// A = SiLU(S) on allowed pairs and the upstream gradient dO of O = A V:
//
//   dA = dO V^T,  dS = dA * SiLU'(S) (0 on masked pairs),  dQ = dS K,  dK = dS^T Q,
//   dV = A^T dO,  SiLU'(x) = sigma(x) (1 + x (1 - sigma(x))).
//
// No softmax, so no row statistics: each gradient is a plain sum over pairs, computed
// by two kernels without atomics (deterministic):
//  * attn_bwd_dq_kernel: a workgroup of 4 waves owns 128 query rows (32 per wave, their
//    Q and dO fragments in registers) and streams 32-key tiles of K and V through LDS.
//    Per block: S^T = K Q^T and dA^T = V dO^T (MFMA, transposed so each lane holds 16
//    keys of one query), dS^T elementwise, then dQ^T += K^T dS^T, with the K^T operand
//    read from row-major K by the transposing LDS read.  24 MFMAs per 32 x 32 block.
//  * attn_bwd_dkv_kernel: a workgroup owns 128 key rows (K and V fragments in registers)
//    and streams 32-query tiles of Q and dO.  Per block: S = Q K^T and dA = dO V^T (each
//    lane holds 16 queries of one key), A and dS elementwise, then dV^T += dO^T A and
//    dK^T += Q^T dS through transposing reads of Q and dO.  32 MFMAs per block.
// Both kernels walk the (sequence, 128-row tile) list of the forward's schedule.
// Operands are fp16 (Q, K, V as the forward takes them; dO, A and dS rounded to fp16),
// accumulation fp32; the bias is formed per element from the two tables.
#include "common.h"
#include "kernels.h"

namespace hstu {

namespace {

constexpr int kBwdRows = 32;      // rows per streamed tile
constexpr int kBwdWaves = 4;
constexpr int kBwdThreads = 64 * kBwdWaves;
constexpr int kBwdMaxPos = 1024;
constexpr int kBwdMaxTime = 64;
constexpr float kLog2e = 1.4426950408889634f;

// ds_read_b64_tr_b16: in each 16-lane group, lane 4 j + q gives the address of row j at
// features 4 q .. 4 q + 3 of a 16-feature slice and receives rows 0..3 of feature lane % 16
__device__ __forceinline__ u32x2 tr_read(const unsigned char *p) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  return __builtin_bit_cast(
      u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)p));
}

// LDS pitches: row copies (16-byte fragment reads of one chunk across 32 rows) and
// transposed-read copies (4 rows x 4 feature groups per 16 lanes) of a 32-row tile
template <int DH>
struct BwdLayout {
  static constexpr int ROWP = DH * 2 + 16;
  static constexpr int TRP = DH * 2 + 32;
  static constexpr int KS = DH / 16;   // k-steps over the head dimension
  static constexpr int FT = DH / 32;   // 32-wide feature tiles
  static constexpr int CPR = DH / 8;   // 16-byte chunks per row
};

__device__ __forceinline__ void silu_and_grad(float s, float &a, float &g) {
  const float sig = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-kLog2e * s));
  a = s * sig;
  g = sig * (1.0f + s * (1.0f - sig));
}

// Rows [r0, r0 + 32) of a fp16 matrix (row pitch `stride` elements, head column offset
// already applied) into an LDS row copy and a transposed-read copy; rows >= n are zero.
template <int DH>
__device__ __forceinline__ void stage_f16(const uint16_t *src, int64_t stride, int r0, int n,
                                          unsigned char *row_copy, unsigned char *tr_copy) {
  using L = BwdLayout<DH>;
  for (int c = threadIdx.x; c < kBwdRows * L::CPR; c += kBwdThreads) {
    const int r = c / L::CPR, ch = c % L::CPR;
    u32x4 v = {0, 0, 0, 0};
    if (r0 + r < n) v = *reinterpret_cast<const u32x4 *>(src + (int64_t)(r0 + r) * stride + ch * 8);
    if (row_copy) *reinterpret_cast<u32x4 *>(row_copy + r * L::ROWP + ch * 16) = v;
    if (tr_copy) *reinterpret_cast<u32x4 *>(tr_copy + r * L::TRP + ch * 16) = v;
  }
}

// Same for an fp32 matrix, rounded to fp16 (saturating)
template <int DH>
__device__ __forceinline__ void stage_f32(const float *src, int64_t stride, int r0, int n,
                                          unsigned char *row_copy, unsigned char *tr_copy) {
  using L = BwdLayout<DH>;
  for (int c = threadIdx.x; c < kBwdRows * L::CPR; c += kBwdThreads) {
    const int r = c / L::CPR, ch = c % L::CPR;
    u32x4 v = {0, 0, 0, 0};
    if (r0 + r < n) {
      const f32x4 a = *reinterpret_cast<const f32x4 *>(src + (int64_t)(r0 + r) * stride + ch * 8);
      const f32x4 b = *reinterpret_cast<const f32x4 *>(src + (int64_t)(r0 + r) * stride + ch * 8 + 4);
      v = u32x4{pack_f16_sat(a[0], a[1]), pack_f16_sat(a[2], a[3]), pack_f16_sat(b[0], b[1]),
                pack_f16_sat(b[2], b[3])};
    }
    if (row_copy) *reinterpret_cast<u32x4 *>(row_copy + r * L::ROWP + ch * 16) = v;
    if (tr_copy) *reinterpret_cast<u32x4 *>(tr_copy + r * L::TRP + ch * 16) = v;
  }
}

// Fragment of row (lane % 32) of a row copy for k-step ks: 8 features 16 ks + 8 (lane / 32)
template <int DH>
__device__ __forceinline__ f16x8 row_frag(const unsigned char *row_copy, int lane, int ks) {
  using L = BwdLayout<DH>;
  return as_f16x8(*reinterpret_cast<const u32x4 *>(row_copy + (lane & 31) * L::ROWP +
                                                    (2 * ks + (lane >> 5)) * 16));
}

// Transposed operand for feature tile f and k-step s2 of a 32-row tile: rows
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

// fp32 row of a register fragment: 8 features 16 ks + 8 (lane / 32) of `row`, as fp16
__device__ __forceinline__ f16x8 f32_row_frag(const float *rowp, bool ok, int lane, int ks) {
  if (!ok) return as_f16x8(u32x4{0, 0, 0, 0});
  const float *p = rowp + 16 * ks + 8 * (lane >> 5);
  const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
  const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
  return as_f16x8(u32x4{pack_f16_sat(a[0], a[1]), pack_f16_sat(a[2], a[3]),
                        pack_f16_sat(b[0], b[1]), pack_f16_sat(b[2], b[3])});
}

__device__ __forceinline__ f16x8 f16_row_frag(const uint16_t *rowp, bool ok, int lane, int ks) {
  if (!ok) return as_f16x8(u32x4{0, 0, 0, 0});
  return as_f16x8(*reinterpret_cast<const u32x4 *>(rowp + 16 * ks + 8 * (lane >> 5)));
}

// packs accumulator values v[8 s2 .. 8 s2 + 7] into the fp16 k-step operand
__device__ __forceinline__ f16x8 pack8(const float *v) {
  return as_f16x8(u32x4{pack_f16(v[0], v[1]), pack_f16(v[2], v[3]), pack_f16(v[4], v[5]),
                        pack_f16(v[6], v[7])});
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

template <int DH>
__global__ __launch_bounds__(kBwdThreads, 2) void attn_bwd_dq_kernel(AttnBwdArgs p) {
  using L = BwdLayout<DH>;
  constexpr int KS = L::KS, FT = L::FT;
  __shared__ __attribute__((aligned(16))) unsigned char k_row[kBwdRows * L::ROWP];
  __shared__ __attribute__((aligned(16))) unsigned char k_tr[kBwdRows * L::TRP];
  __shared__ __attribute__((aligned(16))) unsigned char v_row[kBwdRows * L::ROWP];
  __shared__ int32_t k_ts[kBwdRows];
  __shared__ float ptab[kBwdMaxPos], ttab[kBwdMaxTime];

  const int item = blockIdx.x;
  if (item >= *p.n_work) return;
  const int h = blockIdx.y;
  const int b = p.work[2 * item], qt = p.work[2 * item + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lrow = lane & 31, half = lane >> 5;
  const int s0 = p.offsets[b], n = p.offsets[b + 1] - s0;
  const int rrow = p.rab_per_head ? h : 0;
  BiasCtx bc{ptab, ttab, p.pos_buckets, p.time_buckets, p.rab_pos != nullptr,
             p.rab_time != nullptr && p.ts != nullptr};
  if (bc.use_pos)
    for (int i = tid; i < p.pos_buckets; i += kBwdThreads) ptab[i] = p.rab_pos[rrow * p.pos_buckets + i];
  if (bc.use_time)
    for (int i = tid; i < p.time_buckets; i += kBwdThreads) ttab[i] = p.rab_time[rrow * p.time_buckets + i];

  const int q0 = qt * 128;
  const int qbase = q0 + wave * 32;
  const int qi = qbase + lrow;
  const bool q_ok = qi < n;
  const int32_t qts = bc.use_time ? p.ts[s0 + (q_ok ? qi : 0)] : 0;
  f16x8 qf[KS], dof[KS];
  {
    const uint16_t *qr = p.q + (int64_t)(s0 + qi) * p.stride + h * DH;
    const float *dr = p.d_out + (int64_t)(s0 + qi) * p.d_stride + h * DH;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks] = f16_row_frag(qr, q_ok, lane, ks);
      dof[ks] = f32_row_frag(dr, q_ok, lane, ks);
    }
  }
  f32x16 acc[FT];
#pragma unroll
  for (int f = 0; f < FT; ++f) acc[f] = f32x16{};

  const int k_end = min(n, q0 + 128);  // keys j <= i < q0 + 128
  for (int j0 = 0; j0 < k_end; j0 += kBwdRows) {
    __syncthreads();  // the previous tile is no longer read (and the tables are written)
    stage_f16<DH>(p.k + (int64_t)s0 * p.stride + h * DH, p.stride, j0, n, k_row, k_tr);
    stage_f16<DH>(p.v + (int64_t)s0 * p.stride + h * DH, p.stride, j0, n, v_row, nullptr);
    if (tid < kBwdRows) k_ts[tid] = (bc.use_time && j0 + tid < n) ? p.ts[s0 + j0 + tid] : 0;
    __syncthreads();
    if (j0 > qbase + 31) continue;  // the whole tile is after this wave's queries
    // S^T (bias first) and dA^T; lane: query lrow, keys 8 (i / 4) + 4 half + i % 4
    f32x16 s, da = f32x16{};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kj = j0 + 8 * (i >> 2) + 4 * half + (i & 3);
      s[i] = rab(bc, qi, kj, qts, k_ts[8 * (i >> 2) + 4 * half + (i & 3)]);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s = mfma32_f16(row_frag<DH>(k_row, lane, ks), qf[ks], s);
      da = mfma32_f16(row_frag<DH>(v_row, lane, ks), dof[ks], da);
    }
    float ds[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kj = j0 + 8 * (i >> 2) + 4 * half + (i & 3);
      float a, g;
      silu_and_grad(s[i], a, g);
      ds[i] = (q_ok && kj <= qi) ? da[i] * g : 0.0f;
    }
    // dQ^T += K^T dS^T over the tile's 32 keys
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const f16x8 bop = pack8(ds + 8 * s2);
#pragma unroll
      for (int f = 0; f < FT; ++f) acc[f] = mfma32_f16(tr_frag<DH>(k_tr, lane, f, s2), bop, acc[f]);
    }
  }
  if (q_ok) {
    float *orow = p.dq + (int64_t)(s0 + qi) * p.g_stride + h * DH + half * 4;
#pragma unroll
    for (int f = 0; f < FT; ++f)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<f32x4 *>(orow + f * 32 + g * 8) =
            f32x4{acc[f][4 * g], acc[f][4 * g + 1], acc[f][4 * g + 2], acc[f][4 * g + 3]};
  }
}

template <int DH>
__global__ __launch_bounds__(kBwdThreads, DH == 128 ? 1 : 2) void attn_bwd_dkv_kernel(AttnBwdArgs p) {
  using L = BwdLayout<DH>;
  constexpr int KS = L::KS, FT = L::FT;
  __shared__ __attribute__((aligned(16))) unsigned char q_row[kBwdRows * L::ROWP];
  __shared__ __attribute__((aligned(16))) unsigned char q_tr[kBwdRows * L::TRP];
  __shared__ __attribute__((aligned(16))) unsigned char d_row[kBwdRows * L::ROWP];
  __shared__ __attribute__((aligned(16))) unsigned char d_tr[kBwdRows * L::TRP];
  __shared__ int32_t q_ts[kBwdRows];
  __shared__ float ptab[kBwdMaxPos], ttab[kBwdMaxTime];

  const int item = blockIdx.x;
  if (item >= *p.n_work) return;
  const int h = blockIdx.y;
  const int b = p.work[2 * item];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lrow = lane & 31, half = lane >> 5;
  const int s0 = p.offsets[b], n = p.offsets[b + 1] - s0;
  // the list is ordered for the query tiles (tile t visits t + 1 key tiles); key tile
  // nt - 1 - t visits as many query tiles, so the reversal keeps the longest items first
  const int kt = (n + 127) / 128 - 1 - p.work[2 * item + 1];
  const int rrow = p.rab_per_head ? h : 0;
  BiasCtx bc{ptab, ttab, p.pos_buckets, p.time_buckets, p.rab_pos != nullptr,
             p.rab_time != nullptr && p.ts != nullptr};
  if (bc.use_pos)
    for (int i = tid; i < p.pos_buckets; i += kBwdThreads) ptab[i] = p.rab_pos[rrow * p.pos_buckets + i];
  if (bc.use_time)
    for (int i = tid; i < p.time_buckets; i += kBwdThreads) ttab[i] = p.rab_time[rrow * p.time_buckets + i];

  const int k0 = kt * 128;
  const int kbase = k0 + wave * 32;
  const int kj = kbase + lrow;
  const bool k_ok = kj < n;
  const int32_t kts = bc.use_time ? p.ts[s0 + (k_ok ? kj : 0)] : 0;
  f16x8 kf[KS], vf[KS];
  {
    const uint16_t *kr = p.k + (int64_t)(s0 + kj) * p.stride + h * DH;
    const uint16_t *vr = p.v + (int64_t)(s0 + kj) * p.stride + h * DH;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kf[ks] = f16_row_frag(kr, k_ok, lane, ks);
      vf[ks] = f16_row_frag(vr, k_ok, lane, ks);
    }
  }
  f32x16 dk_acc[FT], dv_acc[FT];
#pragma unroll
  for (int f = 0; f < FT; ++f) dk_acc[f] = dv_acc[f] = f32x16{};

  // queries i >= k0 see these keys; tiles of 32 from the first one
  for (int i0 = k0; i0 < n; i0 += kBwdRows) {
    __syncthreads();
    stage_f16<DH>(p.q + (int64_t)s0 * p.stride + h * DH, p.stride, i0, n, q_row, q_tr);
    stage_f32<DH>(p.d_out + (int64_t)s0 * p.d_stride + h * DH, p.d_stride, i0, n, d_row, d_tr);
    if (tid < kBwdRows) q_ts[tid] = (bc.use_time && i0 + tid < n) ? p.ts[s0 + i0 + tid] : 0;
    __syncthreads();
    if (i0 + 31 < kbase) continue;  // every query of the tile precedes this wave's keys
    // S and dA; lane: key lrow, queries 8 (e / 4) + 4 half + e % 4 of the tile
    f32x16 s, da = f32x16{};
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = 8 * (e >> 2) + 4 * half + (e & 3);
      s[e] = rab(bc, i0 + r, kj, q_ts[r], kts);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s = mfma32_f16(row_frag<DH>(q_row, lane, ks), kf[ks], s);
      da = mfma32_f16(row_frag<DH>(d_row, lane, ks), vf[ks], da);
    }
    float a[16], ds[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int qi = i0 + 8 * (e >> 2) + 4 * half + (e & 3);
      const bool ok = k_ok && qi < n && kj <= qi;
      float av, g;
      silu_and_grad(s[e], av, g);
      a[e] = ok ? av : 0.0f;
      ds[e] = ok ? da[e] * g : 0.0f;
    }
    // dV^T += dO^T A and dK^T += Q^T dS over the tile's 32 queries
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const f16x8 aop = pack8(a + 8 * s2), dop = pack8(ds + 8 * s2);
#pragma unroll
      for (int f = 0; f < FT; ++f) {
        dv_acc[f] = mfma32_f16(tr_frag<DH>(d_tr, lane, f, s2), aop, dv_acc[f]);
        dk_acc[f] = mfma32_f16(tr_frag<DH>(q_tr, lane, f, s2), dop, dk_acc[f]);
      }
    }
  }
  if (k_ok) {
    float *kr = p.dk + (int64_t)(s0 + kj) * p.g_stride + h * DH + half * 4;
    float *vr = p.dv + (int64_t)(s0 + kj) * p.g_stride + h * DH + half * 4;
#pragma unroll
    for (int f = 0; f < FT; ++f)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        *reinterpret_cast<f32x4 *>(kr + f * 32 + g * 8) =
            f32x4{dk_acc[f][4 * g], dk_acc[f][4 * g + 1], dk_acc[f][4 * g + 2], dk_acc[f][4 * g + 3]};
        *reinterpret_cast<f32x4 *>(vr + f * 32 + g * 8) =
            f32x4{dv_acc[f][4 * g], dv_acc[f][4 * g + 1], dv_acc[f][4 * g + 2], dv_acc[f][4 * g + 3]};
      }
  }
}

template <int DH>
hipError_t launch_bwd_dh(const AttnBwdArgs &a, int64_t cap, hipStream_t stream) {
  const dim3 grid((unsigned)cap, (unsigned)a.num_heads);
  attn_bwd_dq_kernel<DH><<<grid, dim3(kBwdThreads), 0, stream>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  attn_bwd_dkv_kernel<DH><<<grid, dim3(kBwdThreads), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention_bwd(const AttnBwdArgs &a, int dh, int64_t cap, hipStream_t stream) {
  if (cap <= 0 || a.num_heads <= 0) return hipSuccess;
  switch (dh) {
    case 32: return launch_bwd_dh<32>(a, cap, stream);
    case 64: return launch_bwd_dh<64>(a, cap, stream);
    case 128: return launch_bwd_dh<128>(a, cap, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace hstu
