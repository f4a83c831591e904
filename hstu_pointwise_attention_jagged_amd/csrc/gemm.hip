// bf16 GEMM with fused epilogue for the two projections of the HSTU layer:
//   f1: UVQK = SiLU(X W1^T + b1)   (equation 1 of the layer), written as fp16
//   f2: Y    = G W2^T + b2         (equation 3), written as bf16
// Both are dense contractions, so they run on MFMA: v_mfma_f32_32x32x16_bf16 with fp32
// accumulation.  Operands are "K-contiguous" (X rows and W rows), staged through LDS
// with a register prefetch of the next K tile (double buffer).  The MFMA takes W as its
// A operand and X as its B operand, so each lane ends with 4 consecutive output columns
// of one token and stores them as one 8-byte bf16 write.
#include "common.h"
#include "kernels.h"

namespace hstu {

namespace {

constexpr int kBK = 64;          // K per stage
constexpr int kPitch = kBK + 8;  // LDS row pitch in bf16 (144 bytes: conflict-free 16B reads)
constexpr int kThreads = 256;

template <int BM, int BN, int ACT, int OUT>
__global__ __launch_bounds__(kThreads, 2) void gemm_kernel(const uint16_t *__restrict__ A,
                                                           const uint16_t *__restrict__ W,
                                                           const float *__restrict__ bias,
                                                           uint16_t *__restrict__ out, int M,
                                                           int N, int K, int n_tiles_n) {
  constexpr int WM = 2, WN = 2;            // waves along tokens / features
  constexpr int TMW = BM / WM, TNW = BN / WN;
  constexpr int MT = TMW / 32, NT = TNW / 32;
  constexpr int A_CHUNKS = BM * kBK / 8 / kThreads;  // 16-byte chunks per thread
  constexpr int W_CHUNKS = BN * kBK / 8 / kThreads;
  static_assert(A_CHUNKS >= 1 && W_CHUNKS >= 1, "tile too small");

  __shared__ __attribute__((aligned(16))) uint16_t xs[2][BM * kPitch];
  __shared__ __attribute__((aligned(16))) uint16_t ws[2][BN * kPitch];

  // feature tile fastest: workgroups that share the X rows are launched together
  const int tile_n = blockIdx.x % n_tiles_n;
  const int tile_m = blockIdx.x / n_tiles_n;
  const int m0 = tile_m * BM, n0 = tile_n * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  u32x4 ra[A_CHUNKS], rw[W_CHUNKS];

  auto load_global = [&](int k0) {
#pragma unroll
    for (int j = 0; j < A_CHUNKS; ++j) {
      const int c = tid + j * kThreads;
      const int row = c / (kBK / 8), col = (c % (kBK / 8)) * 8;
      const int m = m0 + row;
      if (m < M)
        ra[j] = *reinterpret_cast<const u32x4 *>(A + (int64_t)m * K + k0 + col);
      else
        ra[j] = u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < W_CHUNKS; ++j) {
      const int c = tid + j * kThreads;
      const int row = c / (kBK / 8), col = (c % (kBK / 8)) * 8;
      rw[j] = *reinterpret_cast<const u32x4 *>(W + (int64_t)(n0 + row) * K + k0 + col);
    }
  };
  auto store_lds = [&](int buf) {
#pragma unroll
    for (int j = 0; j < A_CHUNKS; ++j) {
      const int c = tid + j * kThreads;
      const int row = c / (kBK / 8), col = (c % (kBK / 8)) * 8;
      *reinterpret_cast<u32x4 *>(&xs[buf][row * kPitch + col]) = ra[j];
    }
#pragma unroll
    for (int j = 0; j < W_CHUNKS; ++j) {
      const int c = tid + j * kThreads;
      const int row = c / (kBK / 8), col = (c % (kBK / 8)) * 8;
      *reinterpret_cast<u32x4 *>(&ws[buf][row * kPitch + col]) = rw[j];
    }
  };

  f32x16 acc[NT][MT];
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int j = 0; j < MT; ++j) acc[i][j] = f32x16{};

  const int nk = K / kBK;
  load_global(0);
  store_lds(0);
  __syncthreads();

  const int lrow = lane & 31, lk = (lane >> 5) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_global((kt + 1) * kBK);
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      bf16x8 wf[NT], xf[MT];
#pragma unroll
      for (int i = 0; i < NT; ++i)
        wf[i] = as_bf16x8(*reinterpret_cast<const u32x4 *>(
            &ws[buf][(wn * TNW + i * 32 + lrow) * kPitch + ks * 16 + lk]));
#pragma unroll
      for (int j = 0; j < MT; ++j)
        xf[j] = as_bf16x8(*reinterpret_cast<const u32x4 *>(
            &xs[buf][(wm * TMW + j * 32 + lrow) * kPitch + ks * 16 + lk]));
#pragma unroll
      for (int i = 0; i < NT; ++i)
#pragma unroll
        for (int j = 0; j < MT; ++j) acc[i][j] = mfma32(wf[i], xf[j], acc[i][j]);
    }
    if (kt + 1 < nk) store_lds(buf ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds token (lane % 32) and features 8g + 4*(lane/32) + 0..3
#pragma unroll
  for (int j = 0; j < MT; ++j) {
    const int m = m0 + wm * TMW + j * 32 + lrow;
    if (m >= M) continue;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * TNW + i * 32 + 8 * g + 4 * (lane >> 5);
        float v0 = acc[i][j][4 * g + 0], v1 = acc[i][j][4 * g + 1];
        float v2 = acc[i][j][4 * g + 2], v3 = acc[i][j][4 * g + 3];
        if (bias != nullptr) {
          const f32x4 bb = *reinterpret_cast<const f32x4 *>(bias + n);
          v0 += bb[0]; v1 += bb[1]; v2 += bb[2]; v3 += bb[3];
        }
        if (ACT == ACT_SILU) {
          v0 = silu_f32(v0); v1 = silu_f32(v1); v2 = silu_f32(v2); v3 = silu_f32(v3);
        }
        u32x2 pk = OUT == OUT_F16 ? u32x2{pack_f16_sat(v0, v1), pack_f16_sat(v2, v3)}
                                  : u32x2{pack_bf16(v0, v1), pack_bf16(v2, v3)};
        *reinterpret_cast<u32x2 *>(out + (int64_t)m * N + n) = pk;
      }
    }
  }
}

template <int BM, int BN, int ACT, int OUT>
hipError_t launch_tile(const uint16_t *A, const uint16_t *W, const float *bias, uint16_t *out,
                       int M, int N, int K, hipStream_t stream) {
  const int tn = N / BN;
  const int tm = (M + BM - 1) / BM;
  gemm_kernel<BM, BN, ACT, OUT><<<dim3(tm * tn), dim3(kThreads), 0, stream>>>(A, W, bias, out, M, N,
                                                                         K, tn);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const uint16_t *A, const uint16_t *W, const float *bias, uint16_t *out,
                       int M, int N, int K, Act act, OutType out_type, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const bool wide = (N % 128) == 0;
  if (act == ACT_SILU && out_type == OUT_F16)
    return wide ? launch_tile<128, 128, ACT_SILU, OUT_F16>(A, W, bias, out, M, N, K, stream)
                : launch_tile<128, 64, ACT_SILU, OUT_F16>(A, W, bias, out, M, N, K, stream);
  if (act == ACT_NONE && out_type == OUT_BF16)
    return wide ? launch_tile<128, 128, ACT_NONE, OUT_BF16>(A, W, bias, out, M, N, K, stream)
                : launch_tile<128, 64, ACT_NONE, OUT_BF16>(A, W, bias, out, M, N, K, stream);
  return hipErrorInvalidValue;
}

}  // namespace hstu
