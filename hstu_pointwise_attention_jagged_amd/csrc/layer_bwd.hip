// Elementwise and reduction kernels of the layer backward: the derivative of equations 1
// and 3 of the layer ("Actions Speak Louder than Words" as retold on chenhuiyu.github.io,
// section "HSTU Layer 到底改了什么") around the attention's own gradient.
//
//  * silu_f16_kernel: U|V|Q|K = SiLU(Z) from the recomputed pre-activations Z (fp16), the
//    operands of the attention that the backward re-forms.
//  * cast_bf16_kernel: the fp32 upstream gradient dY as the bf16 GEMM operand.
//  * norm_gate_bwd_kernel: one wave per row.  From the attention output O (fp32, or rebuilt
//    per head as cn sqrt(var) + mean from the forward's standardised output), the gate U, its
//    pre-activation Z_U and dG = dY w2, it forms N = LayerNorm(O) (two-pass statistics, as
//    the forward), G = N U (bf16, the operand of dw2 = dY^T G), dZ_U = dG N SiLU'(Z_U)
//    (bf16, into the dZ rows) and dO = (dxhat - mean(dxhat) - xhat mean(dxhat xhat)) / sigma
//    with dxhat = dG U gamma (fp32, the attention backward's input).  Each wave walks rows
//    with a grid stride and keeps its column sums of dN xhat and dN (the gamma and beta
//    gradients) in registers, written once as per-wave partials.
//  * colsum kernels: column sums of a row-major matrix in fixed order (per-chunk partials,
//    then one pass over the chunks), so bias gradients are deterministic.
#include "common.h"
#include "kernels.h"

namespace hstu {

namespace {

__device__ __forceinline__ float wave_sum64(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float sigmoid_f32(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * z));
}

// d/dz [z sigma(z)] = sigma (1 + z (1 - sigma))
__device__ __forceinline__ float silu_grad_f32(float z) {
  const float s = sigmoid_f32(z);
  return s * (1.0f + z * (1.0f - s));
}

__global__ __launch_bounds__(256) void silu_f16_kernel(const uint16_t *z, uint16_t *out, int64_t n8) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (int64_t)gridDim.x * 256) {
    const u32x4 v = reinterpret_cast<const u32x4 *>(z)[i];
    u32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a = f16_lo(v[j]), b = f16_hi(v[j]);
      r[j] = pack_f16_sat(a * sigmoid_f32(a), b * sigmoid_f32(b));
    }
    reinterpret_cast<u32x4 *>(out)[i] = r;
  }
}

__global__ __launch_bounds__(256) void cast_bf16_kernel(const float *src, uint16_t *dst, int64_t n4) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    const f32x4 v = reinterpret_cast<const f32x4 *>(src)[i];
    reinterpret_cast<u32x2 *>(dst)[i] = u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
  }
}

constexpr int kNgRows = 4;  // waves (rows in flight) per workgroup

// C: float4 chunks per lane (HDV <= 256 * C); REBUILD: O comes from cn and the head stats
template <int C, bool REBUILD>
__global__ __launch_bounds__(64 * kNgRows) void norm_gate_bwd_kernel(NormGateBwdArgs p) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * kNgRows + (threadIdx.x >> 6);
  const int n_waves = gridDim.x * kNgRows;
  const int HDV = p.hdv;
  const float inv_n = 1.0f / (float)HDV;
  f32x4 sg[C], sb[C];  // this wave's column sums of dN xhat and dN
#pragma unroll
  for (int c = 0; c < C; ++c) sg[c] = sb[c] = f32x4{0, 0, 0, 0};
  for (int row = wave; row < p.T; row += n_waves) {
    const float *grow = p.dg + (int64_t)row * HDV;
    const uint16_t *urow = p.u + (int64_t)row * p.u_stride;
    const uint16_t *zrow = p.zu + (int64_t)row * p.u_stride;
    f32x4 x[C];
    float sum = 0.f;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int e = (lane + 64 * c) * 4;
      x[c] = f32x4{0, 0, 0, 0};
      if (e < HDV) {
        if constexpr (!REBUILD) {
          x[c] = *reinterpret_cast<const f32x4 *>(p.o + (int64_t)row * HDV + e);
        } else {  // the 4 features share a head (dv is a multiple of 32)
          const u32x2 cc = *reinterpret_cast<const u32x2 *>(p.cn + (int64_t)row * HDV + e);
          const float2 st = p.stats[(int64_t)row * (HDV / p.dv) + e / p.dv];
          const float sd = __builtin_amdgcn_sqrtf(st.y);
          x[c] = f32x4{f16_lo(cc[0]) * sd + st.x, f16_hi(cc[0]) * sd + st.x,
                       f16_lo(cc[1]) * sd + st.x, f16_hi(cc[1]) * sd + st.x};
        }
      }
      sum += (x[c][0] + x[c][1]) + (x[c][2] + x[c][3]);
    }
    const float mean = wave_sum64(sum) * inv_n;
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
    const float rstd = 1.0f / sqrtf(wave_sum64(sq) * inv_n + p.eps);
    // xhat in x; dxhat in dx; the row sums of dxhat and dxhat xhat
    f32x4 dx[C];
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int e = (lane + 64 * c) * 4;
      if (e >= HDV) {
        dx[c] = f32x4{0, 0, 0, 0};
        continue;
      }
      const f32x4 dg = *reinterpret_cast<const f32x4 *>(grow + e);
      const u32x2 uu = *reinterpret_cast<const u32x2 *>(urow + e);
      const u32x2 zz = *reinterpret_cast<const u32x2 *>(zrow + e);
      const float u[4] = {f16_lo(uu[0]), f16_hi(uu[0]), f16_lo(uu[1]), f16_hi(uu[1])};
      const float z[4] = {f16_lo(zz[0]), f16_hi(zz[0]), f16_lo(zz[1]), f16_hi(zz[1])};
      float gate[4], dzu[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float xh = (x[c][r] - mean) * rstd;
        x[c][r] = xh;
        const float ga = p.gamma != nullptr ? p.gamma[e + r] : 1.0f;
        const float n = xh * ga + (p.beta != nullptr ? p.beta[e + r] : 0.0f);
        gate[r] = n * u[r];
        dzu[r] = dg[r] * n * silu_grad_f32(z[r]);
        const float dn = dg[r] * u[r];
        sg[c][r] += dn * xh;
        sb[c][r] += dn;
        const float dxh = dn * ga;
        dx[c][r] = dxh;
        s1 += dxh;
        s2 += dxh * xh;
      }
      *reinterpret_cast<u32x2 *>(p.g + (int64_t)row * HDV + e) =
          u32x2{pack_bf16(gate[0], gate[1]), pack_bf16(gate[2], gate[3])};
      *reinterpret_cast<u32x2 *>(p.dzu + (int64_t)row * p.dz_stride + e) =
          u32x2{pack_bf16(dzu[0], dzu[1]), pack_bf16(dzu[2], dzu[3])};
    }
    const float m1 = wave_sum64(s1) * inv_n, m2 = wave_sum64(s2) * inv_n;
    float *dorow = p.d_o + (int64_t)row * HDV;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int e = (lane + 64 * c) * 4;
      if (e >= HDV) continue;
      f32x4 r;
#pragma unroll
      for (int j = 0; j < 4; ++j) r[j] = (dx[c][j] - m1 - x[c][j] * m2) * rstd;
      *reinterpret_cast<f32x4 *>(dorow + e) = r;
    }
  }
  if (p.part_gamma != nullptr || p.part_beta != nullptr) {
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int e = (lane + 64 * c) * 4;
      if (e >= HDV) continue;
      if (p.part_gamma) *reinterpret_cast<f32x4 *>(p.part_gamma + (int64_t)wave * HDV + e) = sg[c];
      if (p.part_beta) *reinterpret_cast<f32x4 *>(p.part_beta + (int64_t)wave * HDV + e) = sb[c];
    }
  }
}

// Column sums of rows [chunk * rows_per, ...) of a [rows][cols] matrix (row pitch stride):
// thread t of block (x, chunk) owns the VEC columns VEC (256 x + t) .. + VEC - 1 and reads
// them with one 16-byte load per row (VEC = 8 bf16 or 4 fp32 values).
template <typename T>
struct Vec16;
template <>
struct Vec16<float> {
  static constexpr int N = 4;
  __device__ static void add(const float *p, float *acc) {
    const f32x4 v = *reinterpret_cast<const f32x4 *>(p);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] += v[j];
  }
};
template <>
struct Vec16<uint16_t> {  // bf16
  static constexpr int N = 8;
  __device__ static void add(const uint16_t *p, float *acc) {
    const u32x4 v = *reinterpret_cast<const u32x4 *>(p);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[2 * j] += __builtin_bit_cast(float, v[j] << 16);
      acc[2 * j + 1] += __builtin_bit_cast(float, v[j] & 0xffff0000u);
    }
  }
};

template <typename T>
__global__ __launch_bounds__(256) void colsum_partial_kernel(const T *a, int rows, int cols,
                                                             int64_t stride, int rows_per,
                                                             float *partial) {
  constexpr int VEC = Vec16<T>::N;
  const int col = (blockIdx.x * 256 + threadIdx.x) * VEC;
  if (col >= cols) return;
  const int r0 = blockIdx.y * rows_per, r1 = min(rows, r0 + rows_per);
  float acc[VEC] = {};
  // unrolled so that several rows' loads are in flight; the adds stay in row order
#pragma unroll 8
  for (int r = r0; r < r1; ++r) Vec16<T>::add(a + (int64_t)r * stride + col, acc);
  float *dst = partial + (int64_t)blockIdx.y * cols + col;
#pragma unroll
  for (int j = 0; j < VEC; ++j) dst[j] = acc[j];
}

// out[col] = sum over k < n_parts of partial[k][col]: 16 threads per column each take
// every 16th part from their first, then the 16 sums are added in a fixed order.
__global__ __launch_bounds__(256) void sum_parts_kernel(const float *partial, int n_parts, int cols,
                                                        float *out) {
  __shared__ float sums[16][17];
  const int c = threadIdx.x & 15, g = threadIdx.x >> 4;
  const int col = blockIdx.x * 16 + c;
  float s = 0.f;
  if (col < cols)
    for (int k = g; k < n_parts; k += 16) s += partial[(int64_t)k * cols + col];
  sums[g][c] = s;
  __syncthreads();
  if (g == 0 && col < cols) {
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) t += sums[i][c];
    out[col] = t;
  }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float *p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[i] = 0.0f;
}

int grid_for(int64_t n) { return (int)(n / 256 + 1 < 2048 ? n / 256 + 1 : 2048); }

}  // namespace

hipError_t launch_fill_zero(float *p, int64_t n, hipStream_t stream) {
  if (p == nullptr || n <= 0) return hipSuccess;
  fill_zero_kernel<<<grid_for(n), 256, 0, stream>>>(p, n);
  return hipGetLastError();
}

hipError_t launch_silu_f16(const uint16_t *z, uint16_t *out, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  silu_f16_kernel<<<grid_for(n / 8), 256, 0, stream>>>(z, out, n / 8);
  return hipGetLastError();
}

hipError_t launch_cast_bf16(const float *src, uint16_t *dst, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  cast_bf16_kernel<<<grid_for(n / 4), 256, 0, stream>>>(src, dst, n / 4);
  return hipGetLastError();
}

int norm_gate_bwd_waves(int T) { return T < kNgWaves ? ((T + kNgRows - 1) / kNgRows) * kNgRows : kNgWaves; }

template <bool REBUILD>
static hipError_t launch_ng(const NormGateBwdArgs &a, int blocks, hipStream_t stream) {
  if (a.hdv <= 256) norm_gate_bwd_kernel<1, REBUILD><<<blocks, 64 * kNgRows, 0, stream>>>(a);
  else if (a.hdv <= 512) norm_gate_bwd_kernel<2, REBUILD><<<blocks, 64 * kNgRows, 0, stream>>>(a);
  else if (a.hdv <= 1024) norm_gate_bwd_kernel<4, REBUILD><<<blocks, 64 * kNgRows, 0, stream>>>(a);
  else norm_gate_bwd_kernel<8, REBUILD><<<blocks, 64 * kNgRows, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_norm_gate_bwd(const NormGateBwdArgs &a, hipStream_t stream) {
  if (a.T <= 0) return hipSuccess;
  const int blocks = norm_gate_bwd_waves(a.T) / kNgRows;
  if (a.o == nullptr) return launch_ng<true>(a, blocks, stream);
  return launch_ng<false>(a, blocks, stream);
}

hipError_t launch_colsum(const void *a, bool bf16, int rows, int cols, int64_t stride,
                         float *partial, int n_parts, float *out, hipStream_t stream) {
  if (cols <= 0) return hipSuccess;
  const int rows_per = (rows + n_parts - 1) / n_parts;
  const int vec = bf16 ? 8 : 4;  // columns per thread; cols is a multiple of 64
  const dim3 grid((cols / vec + 255) / 256, n_parts);
  if (bf16)
    colsum_partial_kernel<uint16_t><<<grid, 256, 0, stream>>>((const uint16_t *)a, rows, cols,
                                                               stride, rows_per, partial);
  else
    colsum_partial_kernel<float><<<grid, 256, 0, stream>>>((const float *)a, rows, cols, stride,
                                                            rows_per, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_sum_parts(partial, n_parts, cols, out, stream);
}

hipError_t launch_sum_parts(const float *partial, int n_parts, int cols, float *out,
                            hipStream_t stream) {
  if (cols <= 0) return hipSuccess;
  sum_parts_kernel<<<(cols + 15) / 16, 256, 0, stream>>>(partial, n_parts, cols, out);
  return hipGetLastError();
}

}  // namespace hstu
