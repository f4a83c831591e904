// Jagged pointwise aggregated attention of the HSTU layer, equation 2:
//     O_h[i] = sum_j SiLU(q_i . k_j + rab^{p,t}(i, j)) v_j
// ("Actions Speak Louder than Words" as retold on chenhuiyu.github.io, section
// "HSTU Layer 到底改了什么"; no softmax and no row normalisation, section
// "不对序列做 softmax"), over keys allowed by a causal or M-FALCON candidate mask, on
// jagged batches computed at their true lengths (section "另外三块拼图", item 1).
//
// gfx950 design
//  * One workgroup = 4 waves = 128 query rows of one (sequence, head); each wave owns 32
//    query rows whose Q fragments stay in registers for the whole key loop.
//  * Keys stream through LDS in stages of 64 (double buffered, register prefetch).  K is
//    stored row-major; V is stored transposed (feature-major) with a key permutation
//    inside each 16-key group, so the MFMA A operand of the P.V product is one 16-byte
//    LDS read per lane.
//  * Scores are computed transposed, S^T = K Q^T (v_mfma_f32_32x32x16_f16), so that each
//    lane's accumulator holds 16 keys of one query; after bias, SiLU and masking these
//    16 values are exactly the lane's B operand (8 keys per k-step) of O^T += V^T P^T,
//    with no trip through LDS.  Q, K, V and A are fp16 operands (the same MFMA rate as
//    bf16 on gfx950, 3 more mantissa bits); accumulation and O stay fp32.
//  * The rab index math is integer only: relative position clamp, and the log2 time
//    bucket from the bit length of (1 + gap); table values come from LDS.
//  * Tiles are skipped from the jagged offsets and the mask: a wave never multiplies a
//    32-key block that lies wholly after its queries (causal) or away from them
//    (candidate self term); only blocks that straddle the diagonal are masked per
//    element.  Masked pairs contribute exactly 0.
#include "common.h"
#include "kernels.h"

namespace hstu {

namespace {

constexpr int kBM = kAttnBlockM;  // 128 queries per workgroup
constexpr int kBN = kAttnBlockN;  // 64 keys per stage
constexpr int kThreads = 256;
constexpr int kMaxPos = 1024;
constexpr int kMaxTime = 64;
constexpr int kVtPitch = kBN + 8;  // transposed V row pitch (fp16): 144 bytes

// Physical slot of key kk (0..63) inside a transposed V stage: within each group of 16
// keys the order is [0-3, 8-11, 4-7, 12-15], which puts the 8 keys a lane multiplies in
// one k-step next to each other.
__device__ __forceinline__ int vt_slot(int kk) {
  const int k = kk & 15;
  return (kk & ~15) + ((k >> 2) & 1) * 8 + (k >> 3) * 4 + (k & 3);
}

template <int DH, int MASK>
__global__ __launch_bounds__(kThreads, 2) void attn_kernel(AttnArgs p) {
  constexpr int KPITCH = DH + 8;        // K row pitch (fp16)
  constexpr int KS = DH / 16;           // k-steps of the score MFMA
  constexpr int FT = DH / 32;           // 32-wide feature tiles of the output
  constexpr int K_CHUNKS = (kBN * DH / 8) / kThreads;  // 16B chunks of K per thread
  constexpr int V_THREADS = 16 * (DH / 8);             // threads staging V (4 keys x 8 feat)
  static_assert(K_CHUNKS >= 1, "DH too small");

  __shared__ __attribute__((aligned(16))) uint16_t ks_lds[2][kBN * KPITCH];
  __shared__ __attribute__((aligned(16))) uint16_t vt_lds[2][DH * kVtPitch];
  __shared__ __attribute__((aligned(16))) int32_t kts_lds[2][kBN];
  __shared__ float ptab[kMaxPos];
  __shared__ float ttab[kMaxTime];

  const int item = blockIdx.x;
  if (item >= *p.n_work) return;
  const int h = blockIdx.y;
  const int b = p.work[2 * item], qt = p.work[2 * item + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lrow = lane & 31, half = lane >> 5;

  const int s0 = p.offsets[b];
  const int n = p.offsets[b + 1] - s0;
  const int q0 = qt * kBM;
  int p0 = 0, n_p = 0;
  if (p.p_offsets != nullptr) {
    p0 = p.p_offsets[b];
    n_p = p.p_offsets[b + 1] - p0;
  }
  const bool use_pos = p.rab_pos != nullptr;
  const bool use_time = p.rab_time != nullptr && p.ts != nullptr &&
                        (p.p_offsets == nullptr || p.p_ts != nullptr);

  // relative-bias tables of this head -> LDS
  {
    const int r = p.rab_per_head ? h : 0;
    if (use_pos)
      for (int i = tid; i < p.pos_buckets; i += kThreads) ptab[i] = p.rab_pos[r * p.pos_buckets + i];
    if (use_time)
      for (int i = tid; i < p.time_buckets; i += kThreads)
        ttab[i] = p.rab_time[r * p.time_buckets + i];
  }

  // this wave's queries: local index qi, position, timestamp; Q fragments in registers
  const int qbase = q0 + wave * 32;
  const int qi = qbase + lrow;
  const bool q_ok = qi < n;
  const int qpos = MASK == 0 ? n_p + qi : n_p;
  const int32_t qts = use_time ? p.ts[s0 + (q_ok ? qi : n - 1)] : 0;
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
  const int q_end = min(n, q0 + kBM);
  const int own_start = MASK == 0 ? 0 : q0;
  const int n_ot = (q_end - own_start + kBN - 1) / kBN;
  const int n_tiles = n_pt + n_ot;

  // staging registers
  u32x4 rk[K_CHUNKS];
  u32x4 rv[4];
  int32_t rts = 0;

  auto tile_src = [&](int t, int &kbase, int &limit, const uint16_t *&kb, const uint16_t *&vb,
                      const int32_t *&tsb, int64_t &stride) {
    if (t < n_pt) {
      kbase = t * kBN;
      limit = n_p;
      kb = p.pk + (int64_t)p0 * p.p_stride;
      vb = p.pv + (int64_t)p0 * p.p_stride;
      tsb = use_time ? p.p_ts + p0 : nullptr;
      stride = p.p_stride;
    } else {
      kbase = own_start + (t - n_pt) * kBN;
      limit = n;
      kb = p.k + (int64_t)s0 * p.stride;
      vb = p.v + (int64_t)s0 * p.stride;
      tsb = use_time ? p.ts + s0 : nullptr;
      stride = p.stride;
    }
  };

  auto load_tile = [&](int t) {
    int kbase, limit;
    const uint16_t *kb, *vb;
    const int32_t *tsb;
    int64_t stride;
    tile_src(t, kbase, limit, kb, vb, tsb, stride);
#pragma unroll
    for (int j = 0; j < K_CHUNKS; ++j) {
      const int c = tid + j * kThreads;
      const int row = c / (DH / 8), col = (c % (DH / 8)) * 8;
      const int key = kbase + row;
      rk[j] = key < limit
                  ? *reinterpret_cast<const u32x4 *>(kb + (int64_t)key * stride + h * DH + col)
                  : u32x4{0, 0, 0, 0};
    }
    if (tid < V_THREADS) {
      const int kg = tid / (DH / 8), fc = (tid % (DH / 8)) * 8;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = kbase + kg * 4 + r;
        rv[r] = key < limit
                    ? *reinterpret_cast<const u32x4 *>(vb + (int64_t)key * stride + h * DH + fc)
                    : u32x4{0, 0, 0, 0};
      }
    }
    if (use_time && tid < kBN) {
      const int key = kbase + tid;
      rts = key < limit ? tsb[key] : 0;
    }
  };

  auto store_tile = [&](int buf) {
#pragma unroll
    for (int j = 0; j < K_CHUNKS; ++j) {
      const int c = tid + j * kThreads;
      const int row = c / (DH / 8), col = (c % (DH / 8)) * 8;
      *reinterpret_cast<u32x4 *>(&ks_lds[buf][row * KPITCH + col]) = rk[j];
    }
    if (tid < V_THREADS) {
      const int kg = tid / (DH / 8), fc = (tid % (DH / 8)) * 8;
      const int slot = vt_slot(kg * 4);
      // transpose 4 keys x 8 features into 8 rows of 4 keys
#pragma unroll
      for (int f = 0; f < 8; ++f) {
        const int w = f >> 1;
        const bool hi = f & 1;
        uint32_t e0 = hi ? (rv[0][w] >> 16) : (rv[0][w] & 0xffffu);
        uint32_t e1 = hi ? (rv[1][w] >> 16) : (rv[1][w] & 0xffffu);
        uint32_t e2 = hi ? (rv[2][w] >> 16) : (rv[2][w] & 0xffffu);
        uint32_t e3 = hi ? (rv[3][w] >> 16) : (rv[3][w] & 0xffffu);
        u32x2 pk = {e0 | (e1 << 16), e2 | (e3 << 16)};
        *reinterpret_cast<u32x2 *>(&vt_lds[buf][(fc + f) * kVtPitch + slot]) = pk;
      }
    }
    if (use_time && tid < kBN) kts_lds[buf][tid] = rts;
  };

  f32x16 acc_o[FT];
#pragma unroll
  for (int f = 0; f < FT; ++f) acc_o[f] = f32x16{};

  if (n_tiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  const int qmin = qbase, qmax = qbase + 31;
  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < n_tiles) load_tile(t + 1);

    const bool is_prefix = t < n_pt;
    const int kbase = is_prefix ? t * kBN : own_start + (t - n_pt) * kBN;
    const int limit = is_prefix ? n_p : n;

#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int k0 = kbase + kb * 32;
      if (k0 >= limit) continue;  // wave-uniform: no valid key in this block
      bool need_mask = false;
      if (!is_prefix) {
        if (MASK == 0) {
          if (k0 > qmax) continue;
          need_mask = k0 + 31 > qmin;
        } else {
          if (k0 > qmax || k0 + 31 < qmin) continue;
          need_mask = true;
        }
      }
      // S^T = K Q^T : lane holds query lrow, keys 8*(i/4) + 4*half + (i%4)
      f32x16 s = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const f16x8 kf = as_f16x8(*reinterpret_cast<const u32x4 *>(
            &ks_lds[buf][(kb * 32 + lrow) * KPITCH + ks * 16 + half * 8]));
        s = mfma32_f16(kf, qf[ks], s);
      }
      float a[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int kl = kb * 32 + 8 * g + 4 * half;  // first of 4 consecutive keys
        int32_t kt4[4] = {0, 0, 0, 0};
        if (use_time) {
          const int4 t4 = *reinterpret_cast<const int4 *>(&kts_lds[buf][kl]);
          kt4[0] = t4.x; kt4[1] = t4.y; kt4[2] = t4.z; kt4[3] = t4.w;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 4 * g + r;
          const int kidx = kbase + kl + r;
          float x = s[i];
          if (use_pos) {
            const int kpos = is_prefix ? kidx : (MASK == 0 ? n_p + kidx : n_p);
            const int rel = max(qpos - kpos, 0);
            x += ptab[min(rel, p.pos_buckets - 1)];
          }
          if (use_time) {
            const int tb = min(time_log2_bucket(qts, kt4[r]), p.time_buckets - 1);
            x += ttab[tb];
          }
          float y = silu_f32(x);
          if (need_mask) {
            const bool allowed = MASK == 0 ? (kidx <= qi) : (kidx == qi);
            y = allowed ? y : 0.0f;
          }
          a[i] = y;
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
      for (int f = 0; f < FT; ++f) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const f16x8 vf = as_f16x8(*reinterpret_cast<const u32x4 *>(
              &vt_lds[buf][(f * 32 + lrow) * kVtPitch + kb * 32 + s2 * 16 + half * 8]));
          acc_o[f] = mfma32_f16(vf, pf[s2], acc_o[f]);
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
// Jagged schedule: one workgroup builds the (sequence, q-tile) list, ordered by the
// number of key tiles each item visits, largest first, with a counting sort.
// ------------------------------------------------------------------------------------
constexpr int kSchedThreads = 1024;
constexpr int kSchedBins = 4096;

__device__ __forceinline__ int item_cost(int n, int n_p, int t, int mask) {
  const int q0 = t * kBM;
  const int q_end = min(n, q0 + kBM);
  const int own = mask == 0 ? q_end : q_end - q0;
  return (n_p + kBN - 1) / kBN + (own + kBN - 1) / kBN;
}

__global__ __launch_bounds__(kSchedThreads) void schedule_kernel(const int32_t *offsets,
                                                                 const int32_t *p_offsets,
                                                                 int B, int mask, int nbins,
                                                                 int32_t *work, int32_t *n_work) {
  __shared__ int bins[kSchedBins];
  __shared__ int total;
  const int tid = threadIdx.x;
  for (int i = tid; i < nbins; i += kSchedThreads) bins[i] = 0;
  __syncthreads();
  for (int b = tid; b < B; b += kSchedThreads) {
    const int n = offsets[b + 1] - offsets[b];
    const int n_p = p_offsets ? p_offsets[b + 1] - p_offsets[b] : 0;
    const int nq = (n + kBM - 1) / kBM;
    for (int t = 0; t < nq; ++t) atomicAdd(&bins[min(item_cost(n, n_p, t, mask), nbins - 1)], 1);
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
    const int nq = (n + kBM - 1) / kBM;
    for (int t = 0; t < nq; ++t) {
      const int pos = atomicAdd(&bins[min(item_cost(n, n_p, t, mask), nbins - 1)], 1);
      work[2 * pos] = b;
      work[2 * pos + 1] = t;
    }
  }
  if (tid == 0) *n_work = total;
}

template <int DH>
hipError_t launch_dh(const AttnArgs &a, int64_t cap, hipStream_t stream) {
  const dim3 grid((unsigned)cap, (unsigned)a.num_heads);
  if (a.mask == 0)
    attn_kernel<DH, 0><<<grid, dim3(kThreads), 0, stream>>>(a);
  else
    attn_kernel<DH, 1><<<grid, dim3(kThreads), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_schedule(const int32_t *offsets, const int32_t *p_offsets, int B, int mask,
                           int max_seq_len, int max_prefix_len, int32_t *work, int32_t *n_work,
                           hipStream_t stream) {
  const int64_t max_cost = (int64_t)(max_prefix_len + kBN - 1) / kBN + (max_seq_len + kBN - 1) / kBN + 1;
  const int nbins = (int)(max_cost < kSchedBins ? max_cost : kSchedBins);
  schedule_kernel<<<1, kSchedThreads, 0, stream>>>(offsets, p_offsets, B, mask, nbins, work, n_work);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs &a, int dh, int64_t cap, hipStream_t stream) {
  if (cap <= 0 || a.num_heads <= 0) return hipSuccess;
  switch (dh) {
    case 32: return launch_dh<32>(a, cap, stream);
    case 64: return launch_dh<64>(a, cap, stream);
    case 128: return launch_dh<128>(a, cap, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace hstu
