// Norm(A(X)V) (.) U of the HSTU layer, equation 3 ("Actions Speak Louder than Words" as
// retold on chenhuiyu.github.io, section "HSTU Layer 到底改了什么"; the LayerNorm that
// follows the unnormalised aggregation, section "不对序列做 softmax"; the gate that
// replaces the feed-forward block, section "用门控代替独立 FFN").
//
// One wave per token row: the fp32 attention output row (H*dv values) is held in
// registers, mean and biased variance come from two wave reductions (two-pass, so the
// large row mean of an unnormalised aggregation does not cancel digits), then the
// normalised value times gamma plus beta is multiplied by the fp16 gate U and written
// as bf16 (the f2 operand).  HBM-bound: 4 B + 2 B read, 2 B written per element.
#include "common.h"
#include "kernels.h"

namespace hstu {

namespace {

constexpr int kRowsPerBlock = 4;

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <int C>  // float4 chunks per lane (HDV <= 256 * C)
__global__ __launch_bounds__(64 * kRowsPerBlock) void norm_gate_kernel(
    const float *__restrict__ O, const uint16_t *__restrict__ U, int64_t u_stride,
    const float *__restrict__ gamma, const float *__restrict__ beta, float eps,
    uint16_t *__restrict__ G, int T, int HDV) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= T) return;
  const float *orow = O + (int64_t)row * HDV;
  f32x4 x[C];
  float sum = 0.f;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int e = (lane + 64 * c) * 4;
    x[c] = e < HDV ? *reinterpret_cast<const f32x4 *>(orow + e) : f32x4{0, 0, 0, 0};
    sum += (x[c][0] + x[c][1]) + (x[c][2] + x[c][3]);
  }
  const float inv_n = 1.0f / (float)HDV;
  const float mean = wave_sum(sum) * inv_n;
  float sq = 0.f;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int e = (lane + 64 * c) * 4;
    if (e < HDV) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float d = x[c][r] - mean;
        sq += d * d;
      }
    }
  }
  const float var = wave_sum(sq) * inv_n;
  const float rstd = 1.0f / sqrtf(var + eps);
  const uint16_t *urow = U + (int64_t)row * u_stride;
  uint16_t *grow = G + (int64_t)row * HDV;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int e = (lane + 64 * c) * 4;
    if (e >= HDV) continue;
    const u32x2 uu = *reinterpret_cast<const u32x2 *>(urow + e);
    float u[4] = {f16_lo(uu[0]), f16_hi(uu[0]), f16_lo(uu[1]), f16_hi(uu[1])};
    float g[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float nv = (x[c][r] - mean) * rstd;
      if (gamma != nullptr) nv *= gamma[e + r];
      if (beta != nullptr) nv += beta[e + r];
      g[r] = nv * u[r];
    }
    u32x2 pk = {pack_bf16(g[0], g[1]), pack_bf16(g[2], g[3])};
    *reinterpret_cast<u32x2 *>(grow + e) = pk;
  }
}

template <int C>
hipError_t launch_c(const float *O, const uint16_t *U, int64_t u_stride, const float *gamma,
                    const float *beta, float eps, uint16_t *G, int T, int HDV, hipStream_t stream) {
  const int blocks = (T + kRowsPerBlock - 1) / kRowsPerBlock;
  norm_gate_kernel<C><<<blocks, 64 * kRowsPerBlock, 0, stream>>>(O, U, u_stride, gamma, beta, eps,
                                                                 G, T, HDV);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_norm_gate(const float *O, const uint16_t *U, int64_t u_stride,
                            const float *gamma, const float *beta, float eps, uint16_t *G,
                            int T, int HDV, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  if (HDV <= 256) return launch_c<1>(O, U, u_stride, gamma, beta, eps, G, T, HDV, stream);
  if (HDV <= 512) return launch_c<2>(O, U, u_stride, gamma, beta, eps, G, T, HDV, stream);
  if (HDV <= 1024) return launch_c<4>(O, U, u_stride, gamma, beta, eps, G, T, HDV, stream);
  if (HDV <= 2048) return launch_c<8>(O, U, u_stride, gamma, beta, eps, G, T, HDV, stream);
  return hipErrorInvalidValue;
}

}  // namespace hstu
