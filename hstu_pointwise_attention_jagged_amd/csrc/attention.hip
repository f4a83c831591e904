// Jagged pointwise aggregated attention of the HSTU layer, equation 2:
//     O_h[i] = sum_j SiLU(q_i . k_j + rab^{p,t}(i, j)) v_j
// ("Actions Speak Louder than Words" as retold on chenhuiyu.github.io, section
// "HSTU Layer 到底改了什么"; no softmax and no row normalisation, section
// "不对序列做 softmax"), over keys allowed by a causal or M-FALCON candidate mask, on
// jagged batches computed at their true lengths (section "另外三块拼图", item 1).
//
// gfx950 design
//  * One workgroup = 4 or 8 waves = 128 or 256 query rows of one (sequence, head); each
//    wave owns 32 query rows whose Q fragments stay in registers for the whole key loop.
//  * Keys stream through LDS in stages of 64 (double buffered, register prefetch through
//    range-checked buffer loads, so keys past a sequence's end read as zero).  K is
//    stored row-major; V is stored transposed (feature-major) with a key permutation
//    inside each 16-key group, so the MFMA A operand of the P.V product is one 16-byte
//    LDS read per lane.
//  * Scores are computed transposed, S^T = K Q^T (v_mfma_f32_32x32x16_f16), so that each
//    lane's accumulator holds 16 keys of one query; after bias, SiLU and masking these
//    16 values are exactly the lane's B operand (8 keys per k-step) of O^T += V^T P^T,
//    with no trip through LDS.  Q, K, V and A are fp16 operands (the same MFMA rate as
//    bf16 on gfx950, 3 more mantissa bits); accumulation and O stay fp32.
//  * The rab index math is integer only: relative position clamp, and the log2 time
//    bucket from the bit length of (1 + gap).  Each wave classifies every 32-key block
//    with scalar arithmetic, from its queries' position / timestamp range and the key
//    block's timestamp range (precomputed by block_stats_kernel):
//      - constant bias: every relative position is past the last position bucket and
//        (the bucket being monotone in the gap) the smallest and largest gap share one
//        time bucket; the score MFMA then starts from that constant;
//      - two buckets: positions as above, gaps spanning exactly buckets b and b+1; one
//        integer compare per element picks between two constants;
//      - general: per-element indices with table values from LDS.
//  * Tiles are skipped from the jagged offsets and the mask: a wave never multiplies a
//    32-key block that lies wholly after its queries (causal) or away from them
//    (candidate self term); only blocks that straddle the diagonal are masked per
//    element.  Masked pairs contribute exactly 0.
//  * When both 32-key blocks of a stage take the constant-bias path, they run as one
//    basic block so the compiler interleaves the MFMAs of one with the SiLU of the other.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace hstu {

namespace {

constexpr int kBN = kAttnBlockN;  // 64 keys per stage
constexpr int kMaxPos = 1024;
constexpr int kMaxTime = 64;
constexpr int kVtPitch = kBN + 8;  // transposed V row pitch (fp16): 144 bytes
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit data format

enum BiasKind { BIAS_CONST = 0, BIAS_TWO = 1, BIAS_GENERAL = 2 };

// Physical slot of key kk (0..63) inside a transposed V stage: within each group of 16
// keys the order is [0-3, 8-11, 4-7, 12-15], which puts the 8 keys a lane multiplies in
// one k-step next to each other.
__device__ __forceinline__ int vt_slot(int kk) {
  const int k = kk & 15;
  return (kk & ~15) + ((k >> 2) & 1) * 8 + (k >> 3) * 4 + (k & 3);
}

// Buffer resource over `bytes` bytes at `base`: loads past the end return 0, so rows
// beyond a sequence's last key are zero without any branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, kRsrcWord3);
}

__device__ __forceinline__ int sgpr(int v) { return __builtin_amdgcn_readfirstlane(v); }

// (gap >= thr) for gap = max(0, ts_q - ts_k) over the full int32 range, thr >= 1.
__device__ __forceinline__ bool gap_at_least(int32_t ts_q, int32_t ts_k, uint32_t thr) {
  return ts_q > ts_k && (uint32_t)ts_q - (uint32_t)ts_k >= thr;
}

template <int DH, int MASK, int NW>
__global__ __launch_bounds__(64 * NW, 2) void attn_kernel(AttnArgs p) {
  constexpr int NT = 64 * NW;           // threads per workgroup
  constexpr int BM = 32 * NW;           // query rows per workgroup
  constexpr int KPITCH = DH + 8;        // K row pitch (fp16)
  constexpr int KS = DH / 16;           // k-steps of the score MFMA
  constexpr int FT = DH / 32;           // 32-wide feature tiles of the output
  constexpr int K_UNITS = kBN * DH / 8;  // 16-byte chunks of a K stage
  constexpr int K_ITERS = (K_UNITS + NT - 1) / NT;
  // V is staged in units of KPU keys x 8 features: 2 keys when that spreads a stage over
  // all threads of an 8-wave group, else 4
  constexpr int KPU = (NW == 8 && (kBN / 2) * (DH / 8) <= NT) ? 2 : 4;
  constexpr int V_GROUPS = kBN / KPU;
  constexpr int V_UNITS = V_GROUPS * (DH / 8);
  static_assert(V_UNITS <= NT, "one V unit per thread");

  __shared__ __attribute__((aligned(16))) uint16_t ks_lds[2][kBN * KPITCH];
  __shared__ __attribute__((aligned(16))) uint16_t vt_lds[2][DH * kVtPitch];
  __shared__ __attribute__((aligned(16))) int32_t kts_lds[2][kBN];
  __shared__ float ptab[kMaxPos];
  __shared__ float ttab[kMaxTime];

  const int item = blockIdx.x;
  if (item >= *p.n_work) return;
  const int h = blockIdx.y;
  const int b = p.work[2 * item], qt = p.work[2 * item + 1];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = sgpr(tid >> 6);
  const int lrow = lane & 31, half = lane >> 5;

  const int s0 = p.offsets[b];
  const int n = p.offsets[b + 1] - s0;
  const int q0 = qt * BM;
  int p0 = 0, n_p = 0;
  if (p.p_offsets != nullptr) {
    p0 = p.p_offsets[b];
    n_p = p.p_offsets[b + 1] - p0;
  }
  const bool use_pos = p.rab_pos != nullptr;
  const bool use_time = p.rab_time != nullptr && p.ts != nullptr &&
                        (p.p_offsets == nullptr || p.p_ts != nullptr);
  const int rrow = p.rab_per_head ? h : 0;
  const float *rab_pos = use_pos ? p.rab_pos + rrow * p.pos_buckets : nullptr;
  const float *rab_time = use_time ? p.rab_time + rrow * p.time_buckets : nullptr;

  // relative-bias tables of this head -> LDS (for the per-element path)
  if (use_pos)
    for (int i = tid; i < p.pos_buckets; i += NT) ptab[i] = rab_pos[i];
  if (use_time)
    for (int i = tid; i < p.time_buckets; i += NT) ttab[i] = rab_time[i];

  // this wave's queries: local index qi, position, timestamp; Q fragments in registers
  const int qbase = q0 + wave * 32;  // wave-uniform
  const int qi = qbase + lrow;
  const bool q_ok = qi < n;
  const bool wave_has_rows = qbase < n;
  const int qpos = MASK == 0 ? n_p + qi : n_p;
  const int32_t qts = use_time ? p.ts[s0 + (q_ok ? qi : n - 1)] : 0;
  int32_t qts_min = q_ok ? qts : INT32_MAX, qts_max = q_ok ? qts : INT32_MIN;
  if (use_time) {
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) {
      qts_min = min(qts_min, __shfl_xor(qts_min, o, 64));
      qts_max = max(qts_max, __shfl_xor(qts_max, o, 64));
    }
    qts_min = sgpr(qts_min);
    qts_max = sgpr(qts_max);
  }
  const int qpos_min = MASK == 0 ? n_p + qbase : n_p;
  f16x8 qf[KS];
  {
    const uint16_t *qrow = p.q + (int64_t)(s0 + qi) * p.stride + h * DH + half * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 v = q_ok ? *reinterpret_cast<const u32x4 *>(qrow + ks * 16) : u32x4{0, 0, 0, 0};
      qf[ks] = as_f16x8(v);
    }
  }

  // key tiles: prefix tiles first, then own tiles
  const int n_pt = (n_p + kBN - 1) / kBN;
  const int q_end = min(n, q0 + BM);
  const int own_start = MASK == 0 ? 0 : q0;
  const int n_ot = (q_end - own_start + kBN - 1) / kBN;
  const int n_tiles = n_pt + n_ot;

  // buffer resources of the two key segments (prefix rows, own rows)
  const int64_t own_bytes = (int64_t)n * p.stride * 2;
  const int64_t pre_bytes = (int64_t)n_p * p.p_stride * 2;
  const __amdgpu_buffer_rsrc_t k_own = make_rsrc(p.k + (int64_t)s0 * p.stride, (uint32_t)own_bytes);
  const __amdgpu_buffer_rsrc_t v_own = make_rsrc(p.v + (int64_t)s0 * p.stride, (uint32_t)own_bytes);
  const __amdgpu_buffer_rsrc_t t_own = make_rsrc(use_time ? p.ts + s0 : p.offsets, use_time ? 4u * n : 0u);
  __amdgpu_buffer_rsrc_t k_pre = k_own, v_pre = v_own, t_pre = t_own;
  if (n_p > 0) {
    k_pre = make_rsrc(p.pk + (int64_t)p0 * p.p_stride, (uint32_t)pre_bytes);
    v_pre = make_rsrc(p.pv + (int64_t)p0 * p.p_stride, (uint32_t)pre_bytes);
    t_pre = make_rsrc(use_time ? p.p_ts + p0 : p.offsets, use_time ? 4u * n_p : 0u);
  }

  // staging registers
  u32x4 rk[K_ITERS];
  u32x4 rv[KPU];
  int32_t rts = 0;

  // V unit of this thread: key group (fastest, so a transposed LDS write of a wave's
  // lanes covers whole 128-byte rows) and feature chunk
  const int v_kg = tid % V_GROUPS, v_fc = (tid / V_GROUPS) * 8;

  auto load_tile = [&](int t) {
    const bool pre = t < n_pt;
    const int kbase = pre ? t * kBN : own_start + (t - n_pt) * kBN;
    const int64_t stride = pre ? p.p_stride : p.stride;
    const __amdgpu_buffer_rsrc_t kr = pre ? k_pre : k_own;
    const __amdgpu_buffer_rsrc_t vr = pre ? v_pre : v_own;
#pragma unroll
    for (int j = 0; j < K_ITERS; ++j) {
      const int c = tid + j * NT;
      if (K_UNITS % NT == 0 || c < K_UNITS) {
        const int row = c / (DH / 8), col = (c % (DH / 8)) * 8;
        const int off = (int)(((int64_t)(kbase + row) * stride + h * DH + col) * 2);
        rk[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(kr, off, 0, 0));
      }
    }
    if (V_UNITS == NT || tid < V_UNITS) {
#pragma unroll
      for (int r = 0; r < KPU; ++r) {
        const int off = (int)(((int64_t)(kbase + v_kg * KPU + r) * stride + h * DH + v_fc) * 2);
        rv[r] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vr, off, 0, 0));
      }
    }
    if (use_time && tid < kBN)
      rts = __builtin_amdgcn_raw_buffer_load_b32(pre ? t_pre : t_own, (kbase + tid) * 4, 0, 0);
  };

  auto store_tile = [&](int buf) {
#pragma unroll
    for (int j = 0; j < K_ITERS; ++j) {
      const int c = tid + j * NT;
      if (K_UNITS % NT == 0 || c < K_UNITS) {
        const int row = c / (DH / 8), col = (c % (DH / 8)) * 8;
        *reinterpret_cast<u32x4 *>(&ks_lds[buf][row * KPITCH + col]) = rk[j];
      }
    }
    if (V_UNITS == NT || tid < V_UNITS) {
      const int slot = vt_slot(v_kg * KPU);
      // transpose KPU keys x 8 features into 8 rows of KPU keys
#pragma unroll
      for (int f = 0; f < 8; ++f) {
        const int w = f >> 1;
        const bool hi = f & 1;
        uint32_t e[KPU];
#pragma unroll
        for (int r = 0; r < KPU; ++r) e[r] = hi ? (rv[r][w] >> 16) : (rv[r][w] & 0xffffu);
        if constexpr (KPU == 2) {
          *reinterpret_cast<uint32_t *>(&vt_lds[buf][(v_fc + f) * kVtPitch + slot]) = e[0] | (e[1] << 16);
        } else {
          u32x2 pk = {e[0] | (e[1] << 16), e[2] | (e[3] << 16)};
          *reinterpret_cast<u32x2 *>(&vt_lds[buf][(v_fc + f) * kVtPitch + slot]) = pk;
        }
      }
    }
    if (use_time && tid < kBN) kts_lds[buf][tid] = rts;
  };

  f32x16 acc_o[FT];
#pragma unroll
  for (int f = 0; f < FT; ++f) acc_o[f] = f32x16{};

  int cur_buf = 0;

  // One 32-key block of this wave: scores, bias, SiLU, mask, aggregation.  The
  // compile-time kind picks the variant, so the common case carries no per-element
  // index or mask code.
  auto block = [&](int kb, int kbase, bool is_prefix, float bias_lo, float bias_hi, uint32_t thr,
                   auto kind_c, auto masked_c) {
    constexpr int KIND = decltype(kind_c)::value;
    constexpr bool MASKED = decltype(masked_c)::value;
    const int buf_ = cur_buf;
    // S^T = K Q^T : lane holds query lrow, keys 8*(i/4) + 4*half + (i%4)
    f32x16 s;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = KIND == BIAS_GENERAL ? 0.0f : bias_lo;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const f16x8 kf = as_f16x8(*reinterpret_cast<const u32x4 *>(
          &ks_lds[buf_][(kb * 32 + lrow) * KPITCH + ks * 16 + half * 8]));
      s = mfma32_f16(kf, qf[ks], s);
    }
    if constexpr (KIND != BIAS_CONST) {
      const float delta = bias_hi - bias_lo;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int kl = kb * 32 + 8 * g + 4 * half;  // first of 4 consecutive keys
        int4 t4 = {0, 0, 0, 0};
        if (use_time) t4 = *reinterpret_cast<const int4 *>(&kts_lds[buf_][kl]);
        const int32_t kt4[4] = {t4.x, t4.y, t4.z, t4.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 4 * g + r;
          if constexpr (KIND == BIAS_TWO) {
            s[i] += gap_at_least(qts, kt4[r], thr) ? delta : 0.0f;
          } else {
            float x = s[i];
            if (use_pos) {
              const int kidx = kbase + kl + r;
              const int kpos = is_prefix ? kidx : (MASK == 0 ? n_p + kidx : n_p);
              x += ptab[min(max(qpos - kpos, 0), p.pos_buckets - 1)];
            }
            if (use_time) x += ttab[min(time_log2_bucket(qts, kt4[r]), p.time_buckets - 1)];
            s[i] = x;
          }
        }
      }
    }
    float a[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) a[i] = silu_f32(s[i]);
    if constexpr (MASKED) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kidx = kbase + kb * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
        const bool allowed = MASK == 0 ? (kidx <= qi) : (kidx == qi);
        a[i] = allowed ? a[i] : 0.0f;
      }
    }
    // P^T operand: k-step s2 takes values 8*s2 .. 8*s2+7
    f16x8 pf[2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      u32x4 pk = {pack_f16(a[8 * s2 + 0], a[8 * s2 + 1]), pack_f16(a[8 * s2 + 2], a[8 * s2 + 3]),
                  pack_f16(a[8 * s2 + 4], a[8 * s2 + 5]), pack_f16(a[8 * s2 + 6], a[8 * s2 + 7])};
      pf[s2] = as_f16x8(pk);
    }
    // O^T += V^T P^T
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
      for (int f = 0; f < FT; ++f) {
        const f16x8 vf = as_f16x8(*reinterpret_cast<const u32x4 *>(
            &vt_lds[buf_][(f * 32 + lrow) * kVtPitch + kb * 32 + s2 * 16 + half * 8]));
        acc_o[f] = mfma32_f16(vf, pf[s2], acc_o[f]);
      }
    }
  };

  // Both 32-key blocks of a stage with a constant bias and no mask (the common case far
  // from the diagonal), in one basic block: the score MFMAs of block B can overlap the
  // SiLU of block A, and the P.V MFMAs of A the SiLU of B.
  auto pair_const = [&](float bias_a, float bias_b) {
    const int buf_ = cur_buf;
    f32x16 sa, sb;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sa[i] = bias_a;
      sb[i] = bias_b;
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const f16x8 kf = as_f16x8(*reinterpret_cast<const u32x4 *>(
          &ks_lds[buf_][lrow * KPITCH + ks * 16 + half * 8]));
      sa = mfma32_f16(kf, qf[ks], sa);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const f16x8 kf = as_f16x8(*reinterpret_cast<const u32x4 *>(
          &ks_lds[buf_][(32 + lrow) * KPITCH + ks * 16 + half * 8]));
      sb = mfma32_f16(kf, qf[ks], sb);
    }
    f16x8 pa[2], pb[2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      u32x4 pk;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        pk[j] = pack_f16(silu_f32(sa[8 * s2 + 2 * j]), silu_f32(sa[8 * s2 + 2 * j + 1]));
      pa[s2] = as_f16x8(pk);
    }
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      u32x4 pk;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        pk[j] = pack_f16(silu_f32(sb[8 * s2 + 2 * j]), silu_f32(sb[8 * s2 + 2 * j + 1]));
      pb[s2] = as_f16x8(pk);
    }
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int f = 0; f < FT; ++f) {
        const f16x8 vf = as_f16x8(*reinterpret_cast<const u32x4 *>(
            &vt_lds[buf_][(f * 32 + lrow) * kVtPitch + s2 * 16 + half * 8]));
        acc_o[f] = mfma32_f16(vf, pa[s2], acc_o[f]);
      }
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int f = 0; f < FT; ++f) {
        const f16x8 vf = as_f16x8(*reinterpret_cast<const u32x4 *>(
            &vt_lds[buf_][(f * 32 + lrow) * kVtPitch + 32 + s2 * 16 + half * 8]));
        acc_o[f] = mfma32_f16(vf, pb[s2], acc_o[f]);
      }
  };

  if (n_tiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();
  // Make the Q fragments complete on every path into the key loop.  Otherwise the
  // wait-count pass sees the Q loads as possibly in flight at the loop header (the
  // no-tile path skips the staging wait) and puts a full vector-memory drain inside
  // the loop, which then also waits for each next tile's prefetch.  The empty asm
  // only names the registers; it touches no memory.
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) asm("" : "+v"(qf[ks]));

  const float pos_last = use_pos ? ptab[p.pos_buckets - 1] : 0.0f;
  const int qmax = qbase + 31;
  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    cur_buf = buf;
    if (t + 1 < n_tiles) load_tile(t + 1);

    const bool is_prefix = t < n_pt;
    const int kbase = is_prefix ? t * kBN : own_start + (t - n_pt) * kBN;
    const int limit = is_prefix ? n_p : n;
    const int2 *kstat = is_prefix ? p.p_kstat + p0 : p.kstat + s0;

    // classify both 32-key blocks with scalar arithmetic
    bool live[2], masked[2];
    int kind[2];
    float blo[2], bhi[2];
    uint32_t thr[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int k0 = kbase + kb * 32;
      bool lv = k0 < limit && wave_has_rows;
      bool mk = false;
      if (!is_prefix) {
        if (MASK == 0) {
          lv = lv && k0 <= qmax;
          mk = k0 + 31 > qbase;
        } else {
          lv = lv && k0 <= qmax && k0 + 31 >= qbase;
          mk = true;
        }
      }
      live[kb] = lv;
      masked[kb] = mk;
      int kd = BIAS_CONST;
      float lo = 0.0f, hi = 0.0f;
      uint32_t th = 1;
      if (use_pos) {
        const int kpos_max = is_prefix ? k0 + 31 : (MASK == 0 ? n_p + k0 + 31 : n_p);
        if (qpos_min - kpos_max >= p.pos_buckets - 1) {
          lo = hi = pos_last;
        } else {
          kd = BIAS_GENERAL;
        }
      }
      if (use_time && kd != BIAS_GENERAL && lv) {
        const int2 st = kstat[k0];  // (min, max) timestamp of keys k0 .. k0+31
        // wave-uniform bucket indices; the values come from the LDS copy of the table so
        // that no vector-memory wait (which would also drain the next tile's prefetch)
        // sits on this path
        const int tb_lo = sgpr(min(time_log2_bucket(qts_min, st.y), p.time_buckets - 1));
        const int tb_hi = sgpr(min(time_log2_bucket(qts_max, st.x), p.time_buckets - 1));
        lo += ttab[tb_lo];
        hi += ttab[tb_hi];
        if (tb_hi != tb_lo) {
          kd = tb_hi == tb_lo + 1 ? BIAS_TWO : BIAS_GENERAL;
          th = (uint32_t)(((uint64_t)1 << (tb_lo + 1)) - 1);
        }
      }
      kind[kb] = kd;
      blo[kb] = lo;
      bhi[kb] = hi;
      thr[kb] = th;
    }
    if (live[0] && live[1] && kind[0] == BIAS_CONST && kind[1] == BIAS_CONST && !masked[0] &&
        !masked[1]) {
      pair_const(blo[0], blo[1]);
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (!live[kb]) continue;
        const float lo = blo[kb], hi = bhi[kb];
        const uint32_t th = thr[kb];
        if (!masked[kb]) {
          if (kind[kb] == BIAS_CONST)
            block(kb, kbase, is_prefix, lo, hi, th, std::integral_constant<int, BIAS_CONST>{}, std::false_type{});
          else if (kind[kb] == BIAS_TWO)
            block(kb, kbase, is_prefix, lo, hi, th, std::integral_constant<int, BIAS_TWO>{}, std::false_type{});
          else
            block(kb, kbase, is_prefix, lo, hi, th, std::integral_constant<int, BIAS_GENERAL>{}, std::false_type{});
        } else {
          if (kind[kb] == BIAS_CONST)
            block(kb, kbase, is_prefix, lo, hi, th, std::integral_constant<int, BIAS_CONST>{}, std::true_type{});
          else
            block(kb, kbase, is_prefix, lo, hi, th, std::integral_constant<int, BIAS_GENERAL>{}, std::true_type{});
        }
      }
    }

    if (t + 1 < n_tiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds query lrow, features 32f + 8g + 4*half + 0..3 -> fp32 rows
  if (q_ok) {
    float *orow = p.out + (int64_t)(s0 + qi) * p.out_stride + h * DH + half * 4;
#pragma unroll
    for (int f = 0; f < FT; ++f)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 v = {acc_o[f][4 * g], acc_o[f][4 * g + 1], acc_o[f][4 * g + 2], acc_o[f][4 * g + 3]};
        *reinterpret_cast<f32x4 *>(orow + f * 32 + g * 8) = v;
      }
  }
}

// ------------------------------------------------------------------------------------
// Timestamp range of every 32-key block: stat[t] = (min, max) of ts over keys
// [t, min(t + 32, end of t's sequence)).  One workgroup per sequence.
// ------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void block_stats_kernel(const int32_t *__restrict__ ts,
                                                          const int32_t *__restrict__ offsets,
                                                          int2 *__restrict__ stat) {
  const int b = blockIdx.x;
  const int s0 = offsets[b], s1 = offsets[b + 1];
  for (int t = s0 + threadIdx.x; t < s1; t += blockDim.x) {
    const int e = min(t + 32, s1);
    int32_t mn = ts[t], mx = mn;
    for (int j = t + 1; j < e; ++j) {
      const int32_t v = ts[j];
      mn = min(mn, v);
      mx = max(mx, v);
    }
    stat[t] = int2{mn, mx};
  }
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

template <int DH, int NW>
hipError_t launch_dh(const AttnArgs &a, int64_t cap, hipStream_t stream) {
  const dim3 grid((unsigned)cap, (unsigned)a.num_heads);
  if (a.mask == 0)
    attn_kernel<DH, 0, NW><<<grid, dim3(64 * NW), 0, stream>>>(a);
  else
    attn_kernel<DH, 1, NW><<<grid, dim3(64 * NW), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

int attn_block_m(int max_seq_len) { return max_seq_len >= 1024 ? 256 : 128; }

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

hipError_t launch_block_stats(const int32_t *ts, const int32_t *offsets, int B, int2 *stat,
                              hipStream_t stream) {
  if (B <= 0) return hipSuccess;
  block_stats_kernel<<<B, 256, 0, stream>>>(ts, offsets, stat);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs &a, int dh, int max_seq_len, int64_t cap,
                            hipStream_t stream) {
  if (cap <= 0 || a.num_heads <= 0) return hipSuccess;
  const bool wide = attn_block_m(max_seq_len) == 256;
  switch (dh) {
    case 32: return wide ? launch_dh<32, 8>(a, cap, stream) : launch_dh<32, 4>(a, cap, stream);
    case 64: return wide ? launch_dh<64, 8>(a, cap, stream) : launch_dh<64, 4>(a, cap, stream);
    case 128: return wide ? launch_dh<128, 8>(a, cap, stream) : launch_dh<128, 4>(a, cap, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace hstu
