// bf16 GEMM with fused epilogue for the two projections of the HSTU layer:
//   f1: UVQK = SiLU(X W1^T + b1)   (equation 1 of the layer), written as fp16
//   f2: Y    = G W2^T + b2         (equation 3), written as bf16
// Both are dense contractions, so they run on MFMA: v_mfma_f32_32x32x16_bf16 with fp32
// accumulation.  Operands are "K-contiguous" (X rows and W rows).  The MFMA takes W as
// its A operand and X as its B operand, so each lane ends with 4 consecutive output
// columns of one token and stores them as one 8-byte write.
//
// Two tilings:
//  * gemm256_kernel (N a multiple of 256): a 256 x 256 output tile per workgroup of 8
//    waves, each wave 64 tokens x 128 features (8 MFMA tiles, 6 operand reads per k-step).
//    K slices of 64 arrive by direct-to-LDS buffer loads (no VGPR staging; rows past M
//    read as zero) into two LDS stages, one stage ahead, issued beside the MFMAs of the
//    first half of the previous stage; 16-byte chunks are
//    XOR-swizzled by row so the operand reads are bank-conflict free without padding.
//    Operand fragments are double-buffered in registers across k-steps, and workgroup
//    ids are remapped so each XCD works through a contiguous range of tiles.  The
//    finished tile goes back through LDS so that every store writes whole rows.
//  * gemm_kernel (any N multiple of 64): 128 x 128 (or 128 x 64) tiles with register
//    prefetch, for the small shapes.
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

// ---------------------------------------------------------------------------------
// 256 x 256 tiles, direct-to-LDS staging
// ---------------------------------------------------------------------------------
constexpr int kBigTile = 256;
constexpr int kBigThreads = 512;
constexpr int kBigBK = 64;      // K per LDS stage
constexpr int kBigStages = 2;   // ring of stages; loads run kBigStages - 1 stages ahead
constexpr int kCPR = kBigBK / 8;  // 16-byte chunks per row
constexpr uint32_t kRsrcWord3 = 0x00020000u;
constexpr int kOutPitch = kBigTile * 2 + 16;  // bytes per output row staged in LDS

// LDS byte offset of 16-byte chunk c (0..7) of row r in a [rows][64] bf16 stage; the
// chunk is XOR-swizzled by row pair so that 16 lanes reading one chunk of 16
// consecutive rows hit distinct banks.
__device__ __forceinline__ int swz(int r, int c) { return (r * kCPR + (c ^ ((r >> 1) & 7))) * 16; }

// Raw buffer descriptor over `bytes` bytes at `base`, both uniform over the workgroup:
// built from scalar copies, so that the descriptor is scalar (a descriptor the compiler
// cannot prove uniform makes it loop over lanes for every load).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void *base, int bytes) {
  const uint64_t b = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  void *p = (void *)(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(p, 0, __builtin_amdgcn_readfirstlane(bytes), kRsrcWord3);
}

// s_waitcnt vmcnt(n) (n <= 15), not waiting on the other counters.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 16, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((15 << 8) | (7 << 4) | N);
}

template <int ACT, int OUT>
__global__ __launch_bounds__(kBigThreads, 2) void gemm256_kernel(const uint16_t *__restrict__ A,
                                                                  const uint16_t *__restrict__ W,
                                                                  const float *__restrict__ bias,
                                                                  uint16_t *__restrict__ out, int M,
                                                                  int N, int K, int n_tiles_n,
                                                                  int n_tiles_total) {
  constexpr int TM = 64, TN = 128;  // wave tile: tokens x features
  constexpr int MT = TM / 32, NT = TN / 32;
  constexpr int STAGE = kBigTile * kBigBK * 2;  // bytes of one operand stage (32 KB)
  constexpr int SEGS = STAGE / 1024 / (kBigThreads / 64);  // 1 KB segments per wave
  constexpr int LOADS = 2 * SEGS;                           // buffer loads per thread per stage
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  unsigned char *xs = smem;                       // [kBigStages][STAGE]
  unsigned char *wsm = smem + kBigStages * STAGE;  // [kBigStages][STAGE]

  // Workgroups are dealt to the 8 XCDs round-robin; give each XCD a contiguous range of
  // tiles (feature tile fastest) so that the tiles sharing X rows share one L2.
  const int nwg = gridDim.x;
  const int per_xcd = (nwg + 7) / 8;
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int lin = xcd * per_xcd + slot;
  if (slot >= per_xcd || lin >= n_tiles_total) return;
  const int tile_n = lin % n_tiles_n;
  const int tile_m = lin / n_tiles_n;
  const int m0 = tile_m * kBigTile, n0 = tile_n * kBigTile;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 3, wn = wave >> 2;  // 4 wave rows of tokens, 2 of features

  // Descriptors over this tile's own row panels (256 rows of A from m0, 256 rows of W from
  // n0), so that every offset below stays under 256 K 2 bytes (the host keeps K <= 2^21)
  // whatever the number of rows; rows of A past M lie outside the range and read as zero.
  const __amdgpu_buffer_rsrc_t ar = uniform_rsrc(A + (int64_t)m0 * K, min(kBigTile, M - m0) * K * 2);
  const __amdgpu_buffer_rsrc_t wr = uniform_rsrc(W + (int64_t)n0 * K, kBigTile * K * 2);

  // Each wave instruction fills 1 KB of LDS = 8 rows x 8 chunks; lane -> (row, chunk)
  // is fixed by the LDS position, the global chunk is the swizzled one.
  const int lrow8 = lane / kCPR, lchunk = lane % kCPR;
  // load j of this wave for stage kt: X segment j (j < SEGS) or W segment j - SEGS
  auto issue_one = [&](int kt, int j) {
    const int stage = kt % kBigStages, k0 = kt * kBigBK;
    const int seg = (j % SEGS) * 8 + wave;   // 8-row segment of the 256-row tile
    const int r = seg * (64 / kCPR) + lrow8;
    const int c = lchunk ^ ((r >> 1) & 7);  // global chunk stored at lchunk
    if (j < SEGS) {
      const int xoff = (r * K + k0 + c * 8) * 2;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, xs + stage * STAGE + seg * 1024, 16, xoff, 0, 0, 0);
    } else {
      const int woff = (r * K + k0 + c * 8) * 2;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, wsm + stage * STAGE + seg * 1024, 16, woff, 0, 0, 0);
    }
  };
  auto issue = [&](int kt) {
#pragma unroll
    for (int j = 0; j < LOADS; ++j) issue_one(kt, j);
  };

  f32x16 acc[NT][MT];
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int j = 0; j < MT; ++j) acc[i][j] = f32x16{};

  const int nk = K / kBigBK;
  // prologue: stages 0 .. kBigStages-2 in flight
#pragma unroll
  for (int kt = 0; kt < kBigStages - 1; ++kt)
    if (kt < nk) issue(kt);

  const int lrow = lane & 31, lk = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    // stage kt has landed for this wave once at most (stages issued after it) remain
    if constexpr (kBigStages == 2) {
      wait_vmcnt<0>();
    } else {
      const int ahead = min(nk - 1 - kt, kBigStages - 2);
      if (ahead >= 2) wait_vmcnt<2 * LOADS>();
      else if (ahead == 1) wait_vmcnt<LOADS>();
      else wait_vmcnt<0>();
    }
    // stage kt complete for all waves; stage kt-1 free for reuse.  A bare barrier: the
    // wait above already covers this wave's direct-to-LDS loads of stage kt, and the
    // later stages stay in flight.
    __builtin_amdgcn_s_barrier();
    const bool more = kt + kBigStages - 1 < nk;

    const unsigned char *xst = xs + (kt % kBigStages) * STAGE;
    const unsigned char *wst = wsm + (kt % kBigStages) * STAGE;
    // operand fragments double-buffered in registers: k-step ks+1 is read while the
    // MFMAs of k-step ks run
    bf16x8 wf[2][NT], xf[2][MT];
    auto read_frags = [&](int ks, int set) {
      const int c = ks * 2 + lk;
#pragma unroll
      for (int i = 0; i < NT; ++i)
        wf[set][i] = as_bf16x8(*reinterpret_cast<const u32x4 *>(wst + swz(wn * TN + i * 32 + lrow, c)));
#pragma unroll
      for (int j = 0; j < MT; ++j)
        xf[set][j] = as_bf16x8(*reinterpret_cast<const u32x4 *>(xst + swz(wm * TM + j * 32 + lrow, c)));
    };
    read_frags(0, 0);
#pragma unroll
    for (int ks = 0; ks < kBigBK / 16; ++ks) {
      if (ks + 1 < kBigBK / 16) read_frags(ks + 1, (ks + 1) & 1);
      // the next stage's loads go out beside the MFMAs of the first two k-steps (half
      // each) rather than in one burst after the barrier, which stalled every wave of
      // the workgroup on the CU's vector-memory queue at once
      if (ks < 2 && more) {
#pragma unroll
        for (int j = ks * (LOADS / 2); j < (ks + 1) * (LOADS / 2); ++j) issue_one(kt + kBigStages - 1, j);
      }
#pragma unroll
      for (int i = 0; i < NT; ++i)
#pragma unroll
        for (int j = 0; j < MT; ++j) acc[i][j] = mfma32(wf[ks & 1][i], xf[ks & 1][j], acc[i][j]);
    }
  }

  // Epilogue through LDS.  A lane holds token (lane % 32) and features 8g + 4*(lane/32)
  // + 0..3 of each MFMA tile, so direct stores would scatter 8-byte pieces over 32 rows
  // per instruction; instead the finished 16-bit tile is staged in LDS (free once every
  // wave is past its last operand read) and written back as whole 512-byte rows.
  __syncthreads();
#pragma unroll
  for (int j = 0; j < MT; ++j) {
    const int r = wm * TM + j * 32 + lrow;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = wn * TN + i * 32 + 8 * g + 4 * lk;
        float v0 = acc[i][j][4 * g + 0], v1 = acc[i][j][4 * g + 1];
        float v2 = acc[i][j][4 * g + 2], v3 = acc[i][j][4 * g + 3];
        if (bias != nullptr) {
          const f32x4 bb = *reinterpret_cast<const f32x4 *>(bias + n0 + c);
          v0 += bb[0]; v1 += bb[1]; v2 += bb[2]; v3 += bb[3];
        }
        if (ACT == ACT_SILU) {
          v0 = silu_f32(v0); v1 = silu_f32(v1); v2 = silu_f32(v2); v3 = silu_f32(v3);
        }
        const u32x2 pk = OUT == OUT_F16 ? u32x2{pack_f16_sat(v0, v1), pack_f16_sat(v2, v3)}
                                        : u32x2{pack_bf16(v0, v1), pack_bf16(v2, v3)};
        *reinterpret_cast<u32x2 *>(smem + r * kOutPitch + c * 2) = pk;
      }
    }
  }
  __syncthreads();
  // Each wave instruction stores two whole rows of the tile (64 lanes x 16 bytes).  The
  // fp16 products (U, V, Q, K: four times the model width) outgrow the last-level cache
  // and are streamed past it with non-temporal stores, which keeps the operands cached;
  // the bf16 output (the next layer's input) is stored normally.
  constexpr int kRowChunks = kBigTile * 2 / 16;
#pragma unroll
  for (int it = 0; it < kBigTile * kRowChunks / kBigThreads; ++it) {
    const int ch = it * kBigThreads + tid;
    const int r = ch / kRowChunks, c16 = ch % kRowChunks;
    const u32x4 v = *reinterpret_cast<const u32x4 *>(smem + r * kOutPitch + c16 * 16);
    u32x4 *dst = reinterpret_cast<u32x4 *>(out + (int64_t)(m0 + r) * N + n0 + c16 * 8);
    if (m0 + r < M) {
      if constexpr (OUT == OUT_F16) __builtin_nontemporal_store(v, dst);
      else *dst = v;
    }
  }
}

template <int ACT, int OUT>
hipError_t launch_big(const uint16_t *A, const uint16_t *W, const float *bias, uint16_t *out,
                      int M, int N, int K, hipStream_t stream) {
  const int tn = N / kBigTile;
  const int tm = (M + kBigTile - 1) / kBigTile;
  const int total = tm * tn;
  const int grid = (total + 7) / 8 * 8;
  // operand stages (2 operands each), reused for the output tile in the epilogue
  const size_t lds = std::max(2 * (size_t)kBigStages * kBigTile * kBigBK * 2, (size_t)kBigTile * kOutPitch);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void *)gemm256_kernel<ACT, OUT>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  gemm256_kernel<ACT, OUT><<<dim3(grid), dim3(kBigThreads), lds, stream>>>(A, W, bias, out, M, N,
                                                                           K, tn, total);
  return hipGetLastError();
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
  if (K > kGemmMaxK) return hipErrorInvalidValue;  // 32-bit offsets within a 256-row panel
  const bool big = (N % kBigTile) == 0 && M >= kBigTile;
  const bool wide = (N % 128) == 0;
  if (act == ACT_SILU && out_type == OUT_F16) {
    if (big) return launch_big<ACT_SILU, OUT_F16>(A, W, bias, out, M, N, K, stream);
    return wide ? launch_tile<128, 128, ACT_SILU, OUT_F16>(A, W, bias, out, M, N, K, stream)
                : launch_tile<128, 64, ACT_SILU, OUT_F16>(A, W, bias, out, M, N, K, stream);
  }
  if (act == ACT_NONE && out_type == OUT_F16) {  // pre-activations (the backward's recompute)
    if (big) return launch_big<ACT_NONE, OUT_F16>(A, W, bias, out, M, N, K, stream);
    return wide ? launch_tile<128, 128, ACT_NONE, OUT_F16>(A, W, bias, out, M, N, K, stream)
                : launch_tile<128, 64, ACT_NONE, OUT_F16>(A, W, bias, out, M, N, K, stream);
  }
  if (act == ACT_NONE && out_type == OUT_BF16) {
    if (big) return launch_big<ACT_NONE, OUT_BF16>(A, W, bias, out, M, N, K, stream);
    return wide ? launch_tile<128, 128, ACT_NONE, OUT_BF16>(A, W, bias, out, M, N, K, stream)
                : launch_tile<128, 64, ACT_NONE, OUT_BF16>(A, W, bias, out, M, N, K, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace hstu
