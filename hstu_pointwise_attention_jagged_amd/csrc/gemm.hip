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

// Rows present: min(cap, *m_dev), or cap without m_dev.  The count is read through the
// constant address space, so it is a scalar load (the first thing every workgroup waits
// for; a vector load took a full round trip through the vector memory path).
__device__ __forceinline__ int rows_present(const int32_t *m_dev, int cap) {
  return m_dev != nullptr ? min(cap, *(const __attribute__((address_space(4))) int32_t *)m_dev) : cap;
}

constexpr int kBK = 64;          // K per stage
constexpr int kPitch = kBK + 8;  // LDS row pitch in bf16 (144 bytes: conflict-free 16B reads)
constexpr int kThreads = 256;

template <int BM, int BN, int ACT, int OUT>
__global__ __launch_bounds__(kThreads, 2) void gemm_kernel(const uint16_t *__restrict__ A,
                                                           const uint16_t *__restrict__ W,
                                                           const float *__restrict__ bias,
                                                           uint16_t *__restrict__ out,
                                                           const int32_t *__restrict__ m_dev,
                                                           int M_cap, int N, int K, int n_tiles_n) {
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
  const int M = rows_present(m_dev, M_cap);
  if (m0 >= M) return;
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

// s_waitcnt vmcnt(n) (n <= 63: low 4 bits in [3:0], high 2 bits in [15:14]), not waiting
// on the other counters.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(((N >> 4) << 14) | (15 << 8) | (7 << 4) | (N & 15));
}

// Item i of the f2 operand conversion: 8 values of w2 (bf16 -> fp16) and entry i of the
// gamma | beta table.  The caller has set MODE.FP16_OVFL (values past the fp16 range clamp
// to +-65504, as in the f2 kernel).
__device__ __forceinline__ void gate_prep_item(const W2Prep &q, int64_t i) {
  if (i * 8 < q.n_w) {
    const u32x4 v = *reinterpret_cast<const u32x4 *>(q.w2 + i * 8);
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o[e] = pack_f16(__builtin_bit_cast(float, v[e] << 16), __builtin_bit_cast(float, v[e] & 0xffff0000u));
    *reinterpret_cast<u32x4 *>(q.w2h + i * 8) = o;
  }
  if (q.gb != nullptr && i < q.K) {
    q.gb[i] = (_Float16)(q.gamma != nullptr ? q.gamma[i] : 1.0f);
    q.gb[q.K + i] = (_Float16)(q.beta != nullptr ? q.beta[i] : 0.0f);
  }
}

__host__ __device__ inline int64_t gate_prep_work(const W2Prep &q) {
  return std::max<int64_t>((q.n_w + 7) / 8, q.K);
}

// Operand layouts: KC, the operand's rows are the output's rows (or columns) and K is
// contiguous (X [M][K], W [N][K]); KR, the operand's rows are K (X [K][M], W [K][N]).
// A KC stage is [256 rows][64 k] read with 16-byte reads; a KR stage is the natural
// [64 k][256 columns] slice, read with the transposing ds_read_b64_tr_b16, whose lane
// layout is chosen to give the same k order as the 16-byte read, so the two layouts mix.
template <int LX, int LW, int ACT, int OUT>
__global__ __launch_bounds__(kBigThreads, 2) void gemm256_kernel(GemmArgs g) {
  constexpr int TM = 64, TN = 128;  // wave tile: tokens x features
  constexpr int MT = TM / 32, NT = TN / 32;
  constexpr int STAGE = kBigTile * kBigBK * 2;  // bytes of one operand stage (32 KB)
  constexpr int SEGS = STAGE / 1024 / (kBigThreads / 64);  // 1 KB segments per wave
  static_assert(OUT != OUT_F32 || ACT == ACT_NONE, "fp32 output is a plain product");
  if constexpr (ACT == ACT_SILU) {
    // workgroups past the product's grid: the f2 operand conversion (W2Prep); they are
    // dispatched after every tile of the product, so they run in its tail
    if ((int)blockIdx.x >= g.prep.grid_gemm) {
      __builtin_amdgcn_s_setreg((0 << 11) | (23 << 6) | 1, 1);  // MODE.FP16_OVFL
      const int64_t work = gate_prep_work(g.prep);
      for (int64_t i = (int64_t)((int)blockIdx.x - g.prep.grid_gemm) * kBigThreads + threadIdx.x; i < work;
           i += (int64_t)g.prep.blocks * kBigThreads)
        gate_prep_item(g.prep, i);
      return;
    }
  }
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  unsigned char *xs = smem;                       // [kBigStages][STAGE]
  unsigned char *wsm = smem + kBigStages * STAGE;  // [kBigStages][STAGE]
  const int N = g.N;

  // Workgroups are dealt to the 8 XCDs round-robin; give each XCD a contiguous range of
  // the units present (K split, then tile; feature tile fastest) so that the tiles
  // sharing operand panels share one L2.  The range comes from the rows present, which
  // may be fewer than the grid was sized for: the work then still spreads over every XCD,
  // and the surplus workgroups (the highest slots) exit.
  const int M = rows_present(g.m_dev, g.M);
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  int split = 0, m0, n0;
  if (g.splits == 1) {
    // XCD x owns feature tiles [x % xn, +1) x nb and row panels [x / xn, +1) x mh (feature
    // tile fastest): the W panels an XCD uses stay in its L2 while the row panels stream
    // past, each read by xn XCDs
    const int xn = g.xcd_n, nb = g.n_tiles_n / xn;
    const int tm = (M + kBigTile - 1) / kBigTile;
    const int mh = (tm + 8 / xn - 1) / (8 / xn);
    const int m_lo = (xcd / xn) * mh, count = (min(tm, m_lo + mh) - m_lo) * nb;
    if (slot >= count) return;
    m0 = (m_lo + slot / nb) * kBigTile;
    n0 = ((xcd % xn) * nb + slot % nb) * kBigTile;
  } else {
    // splits: each XCD a contiguous range of (split, tile) units, tile fastest
    const int tiles = g.n_tiles_total;
    const int units = tiles * g.splits;
    const int per_xcd = (units + 7) / 8;
    const int lin = xcd * per_xcd + slot;
    if (slot >= per_xcd || lin >= units) return;
    split = lin / tiles;
    const int tl = lin % tiles;
    m0 = (tl / g.n_tiles_n) * kBigTile;
    n0 = (tl % g.n_tiles_n) * kBigTile;
  }
  const int kb = split * g.k_split, ke = min(g.K, kb + g.k_split);
  const int nk = (ke - kb + kBigBK - 1) / kBigBK;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 3, wn = wave >> 2;  // 4 wave rows of tokens, 2 of features

  // Descriptors.  KC: over the tile's 256-row panel (offsets below 256 ld 2 bytes, ld <=
  // 2^21), rows past the matrix read as zero.  KR: over the split's K rows from the
  // tile's first column (offsets below k_split ld 2 bytes <= 2^31), rows past K read as
  // zero; columns past the matrix read whatever follows and only reach output rows or
  // columns that are not stored.
  const __amdgpu_buffer_rsrc_t xr =
      LX == KC ? uniform_rsrc(g.x + (int64_t)m0 * g.ldx, min(kBigTile, M - m0) * (int)g.ldx * 2)
               : uniform_rsrc(g.x + (int64_t)kb * g.ldx + m0, (ke - kb) * (int)g.ldx * 2);
  const __amdgpu_buffer_rsrc_t wr =
      LW == KC ? uniform_rsrc(g.w + (int64_t)n0 * g.ldw, min(kBigTile, N - n0) * (int)g.ldw * 2)
               : uniform_rsrc(g.w + (int64_t)kb * g.ldw + n0, (ke - kb) * (int)g.ldw * 2);
  const int ldx = (int)g.ldx, ldw = (int)g.ldw;

  // Each wave instruction fills 1 KB of LDS.  KC: 8 rows x 8 chunks, lane -> (row lane /
  // 8, chunk lane % 8), the global chunk being the swizzled one.  KR: 2 k rows x 32
  // chunks, lane -> (k row lane / 32, chunk lane % 32), 16-byte chunks XOR-swizzled by
  // 4 (k % 4) so that the transposing reads of 32 lanes hit distinct banks.
  auto issue_op = [&](auto layout, const __amdgpu_buffer_rsrc_t &rs, int ld, unsigned char *dst, int k0,
                      int j) __attribute__((always_inline)) {
    constexpr int L = decltype(layout)::value;
    const int seg = j * 8 + wave;
    if constexpr (L == KC) {
      const int r = seg * (64 / kCPR) + lane / kCPR;
      const int c = (lane % kCPR) ^ ((r >> 1) & 7);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst + seg * 1024, 16, (r * ld + kb + k0 + c * 8) * 2, 0, 0, 0);
    } else {
      const int kr = seg * 2 + (lane >> 5);
      const int c = (lane & 31) ^ ((kr & 3) << 2);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst + seg * 1024, 16, ((k0 + kr) * ld + c * 8) * 2, 0, 0, 0);
    }
  };
  // load j of this wave for stage kt: X segment j (j < SEGS) or W segment j - SEGS
  auto issue_one = [&](int kt, int j) {
    const int stage = kt % kBigStages, k0 = kt * kBigBK;
    if (j < SEGS)
      issue_op(std::integral_constant<int, LX>{}, xr, ldx, xs + stage * STAGE, k0, j);
    else
      issue_op(std::integral_constant<int, LW>{}, wr, ldw, wsm + stage * STAGE, k0, j - SEGS);
  };

  // Per-lane parts of the fragment reads.  KC: 16-byte read of chunk 2 ks + lane / 32 of
  // row (block + lane % 32).  KR: two transposing reads; in each 16-lane group lane 4 j + q
  // names k row 8 (lane / 32) + j (then + 4) at columns 16 ((lane / 16) % 2) + 4 q ..+3 of
  // the 32-column block, and receives the four k values of column lane % 32: k
  // 8 (lane / 32) + 0..7 over the two reads, as the 16-byte read gives.
  const int lrow = lane & 31, lk = lane >> 5;
  const int tr_j = (lane & 15) >> 2;
  const int tr_base = (8 * lk + tr_j) * 512 + (2 * ((lane >> 4) & 1) + ((lane & 3) >> 1)) * 16 + (lane & 1) * 8;
  auto tr_off = [&](int col_block) { return tr_base + (((col_block >> 3) ^ (tr_j << 2)) << 4); };
  int xo[MT], wo[NT];
#pragma unroll
  for (int j = 0; j < MT; ++j) xo[j] = LX == KC ? 0 : tr_off(wm * TM + j * 32);
#pragma unroll
  for (int i = 0; i < NT; ++i) wo[i] = LW == KC ? 0 : tr_off(wn * TN + i * 32);
  auto read_op = [&](auto layout, const unsigned char *st, int row_block, int off, int ks) __attribute__((always_inline)) {
    constexpr int L = decltype(layout)::value;
    if constexpr (L == KC) {
      return as_bf16x8(*reinterpret_cast<const u32x4 *>(st + swz(row_block + lrow, ks * 2 + lk)));
    } else {
      const u32x2 lo = lds_read_tr16(st + ks * 16 * 512 + off);
      const u32x2 hi = lds_read_tr16(st + ks * 16 * 512 + 4 * 512 + off);
      return as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
    }
  };

  f32x16 acc[NT][MT];
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int j = 0; j < MT; ++j) acc[i][j] = f32x16{};

  // prologue: stages 0 .. kBigStages-2 in flight
#pragma unroll
  for (int kt = 0; kt < kBigStages - 1; ++kt)
    if (kt < nk)
#pragma unroll
      for (int j = 0; j < 2 * SEGS; ++j) issue_one(kt, j);

  for (int kt = 0; kt < nk; ++kt) {
    static_assert(kBigStages == 2, "one stage in flight");
    wait_vmcnt<0>();  // this wave's loads of stage kt (the only ones in flight)
    // stage kt complete for all waves; stage kt-1 free for reuse.  A bare barrier: the
    // wait above already covers this wave's direct-to-LDS loads.
    __builtin_amdgcn_s_barrier();
    const bool more = kt + 1 < nk;
    const unsigned char *xst = xs + (kt % kBigStages) * STAGE;
    const unsigned char *wst = wsm + (kt % kBigStages) * STAGE;
    // operand fragments double-buffered in registers: k-step ks+1 is read while the
    // MFMAs of k-step ks run
    bf16x8 wf[2][NT], xf[2][MT];
    auto read_frags = [&](int ks, int set) {
#pragma unroll
      for (int i = 0; i < NT; ++i)
        wf[set][i] = read_op(std::integral_constant<int, LW>{}, wst, wn * TN + i * 32, wo[i], ks);
#pragma unroll
      for (int j = 0; j < MT; ++j)
        xf[set][j] = read_op(std::integral_constant<int, LX>{}, xst, wm * TM + j * 32, xo[j], ks);
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
        for (int j = ks * SEGS; j < (ks + 1) * SEGS; ++j) issue_one(kt + 1, j);
      }
#pragma unroll
      for (int i = 0; i < NT; ++i)
#pragma unroll
        for (int j = 0; j < MT; ++j) acc[i][j] = mfma32(wf[ks & 1][i], xf[ks & 1][j], acc[i][j]);
    }
  }

  // Epilogue through LDS.  A lane holds token (lane % 32) and features 8g + 4*(lane/32)
  // + 0..3 of each MFMA tile, so direct stores would scatter 8-byte pieces over 32 rows
  // per instruction; instead the finished tile is staged in LDS (free once every wave is
  // past its last operand read) and written back as whole rows, 16-byte chunks past N
  // skipped.
  if constexpr (OUT == OUT_F32) {
    // fp32 rows of 1 KB: the tile goes out in two halves of 128 rows (waves 0, 1, 4, 5
    // then 2, 3, 6, 7); with splits, split s writes its own [M][N] slice
    constexpr int kPitch32 = kBigTile * 4 + 16;
    float *out = reinterpret_cast<float *>(g.out) + (int64_t)split * g.M * N;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      __syncthreads();
      if ((wm >> 1) == h) {
#pragma unroll
        for (int j = 0; j < MT; ++j) {
          const int r = (wm & 1) * TM + j * 32 + lrow;
#pragma unroll
          for (int i = 0; i < NT; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int c = wn * TN + i * 32 + 8 * q + 4 * lk;
              *reinterpret_cast<f32x4 *>(smem + r * kPitch32 + c * 4) =
                  f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
            }
        }
      }
      __syncthreads();
      constexpr int kRowChunks = kBigTile * 4 / 16;
#pragma unroll
      for (int it = 0; it < 128 * kRowChunks / kBigThreads; ++it) {
        const int ch = it * kBigThreads + tid;
        const int r = ch / kRowChunks, c16 = ch % kRowChunks;
        const int m = m0 + h * 128 + r, n = n0 + c16 * 4;
        if (m < M && n < N)
          *reinterpret_cast<u32x4 *>(out + (int64_t)m * N + n) =
              *reinterpret_cast<const u32x4 *>(smem + r * kPitch32 + c16 * 16);
      }
    }
  } else {
    uint16_t *out = reinterpret_cast<uint16_t *>(g.out);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < MT; ++j) {
      const int r = wm * TM + j * 32 + lrow;
#pragma unroll
      for (int i = 0; i < NT; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = wn * TN + i * 32 + 8 * q + 4 * lk;
          float v0 = acc[i][j][4 * q + 0], v1 = acc[i][j][4 * q + 1];
          float v2 = acc[i][j][4 * q + 2], v3 = acc[i][j][4 * q + 3];
          if (g.bias != nullptr && n0 + c < N) {
            const f32x4 bb = *reinterpret_cast<const f32x4 *>(g.bias + n0 + c);
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
      if (m0 + r < M && n0 + c16 * 8 < N) {
        if constexpr (OUT == OUT_F16) __builtin_nontemporal_store(v, dst);
        else *dst = v;
      }
    }
  }
}

// out[i] = sum over s (in order) of part[s][i], n a multiple of 4
__global__ __launch_bounds__(256) void sum_splits_kernel(const float *__restrict__ part, int splits,
                                                         int64_t n, float *__restrict__ out) {
  const int64_t n4 = n / 4;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    f32x4 acc = reinterpret_cast<const f32x4 *>(part)[i];
    for (int s = 1; s < splits; ++s) acc += reinterpret_cast<const f32x4 *>(part + (int64_t)s * n)[i];
    reinterpret_cast<f32x4 *>(out)[i] = acc;
  }
}

// XCDs along the feature tiles: the fewest (1, 2, 4 or 8, dividing the feature tile
// count) that keep each XCD's W panels within 2 MB of its 4 MB L2.
static int xcd_split_n(int n_tiles_n, int64_t panel_bytes) {
  for (int xn = 1; xn < 8; xn *= 2)
    if (n_tiles_n % xn == 0 && (int64_t)(n_tiles_n / xn) * panel_bytes <= ((int64_t)2 << 20)) return xn;
  return n_tiles_n % 8 == 0 ? 8 : (n_tiles_n % 4 == 0 ? 4 : (n_tiles_n % 2 == 0 ? 2 : 1));
}

template <int LX, int LW, int ACT, int OUT>
hipError_t launch_big(GemmArgs a, hipStream_t stream) {
  int grid;
  if (a.splits == 1) {
    a.xcd_n = xcd_split_n(a.n_tiles_n, (int64_t)kBigTile * a.K * 2);
    const int tm = (a.M + kBigTile - 1) / kBigTile, xm = 8 / a.xcd_n;
    grid = 8 * ((tm + xm - 1) / xm) * (a.n_tiles_n / a.xcd_n);
  } else {
    grid = (a.n_tiles_total * a.splits + 7) / 8 * 8;
  }
  a.prep.grid_gemm = grid;
  if (ACT == ACT_SILU && a.prep.w2h != nullptr) {
    // the f2 operand conversion: up to 64 more workgroups, about 4 items per thread
    const int64_t work = gate_prep_work(a.prep);
    a.prep.blocks = (int)std::min<int64_t>(64, std::max<int64_t>(1, (work + 4 * kBigThreads - 1) / (4 * kBigThreads)));
    grid += a.prep.blocks;
  }
  // operand stages (2 operands each), reused for the output tile in the epilogue
  const size_t lds = std::max(2 * (size_t)kBigStages * kBigTile * kBigBK * 2,
                              OUT == OUT_F32 ? (size_t)128 * (kBigTile * 4 + 16) : (size_t)kBigTile * kOutPitch);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void *)gemm256_kernel<LX, LW, ACT, OUT>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  gemm256_kernel<LX, LW, ACT, OUT><<<dim3(grid), dim3(kBigThreads), lds, stream>>>(a);
  return hipGetLastError();
}

template <int BM, int BN, int ACT, int OUT>
hipError_t launch_tile(const uint16_t *A, const uint16_t *W, const float *bias, uint16_t *out,
                       int M, int N, int K, hipStream_t stream, const int32_t *m_dev) {
  const int tn = N / BN;
  const int tm = (M + BM - 1) / BM;
  gemm_kernel<BM, BN, ACT, OUT><<<dim3(tm * tn), dim3(kThreads), 0, stream>>>(A, W, bias, out, m_dev,
                                                                         M, N, K, tn);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------
// f2 with LayerNorm and the U gate formed in its operand staging (equation 3:
// Y = f2(LayerNorm(A(X)V) (.) U)).  The attention leaves each head's part of a row
// standardised (c, fp16) with its mean and biased variance; the LayerNorm over the whole
// row is rebuilt exactly from those:  mu = mean of the head means, var = mean of
// (head variance + (head mean - mu)^2), rstd = 1 / sqrt(var + eps), and for a feature of
// head h:  (o - mu) rstd = c a_h + b_h  with  a_h = sqrt(var_h) rstd, b_h = (mu_h - mu) rstd.
// G = ((c a_h + b_h) gamma + beta) U is formed in packed fp16 by the thread that stages it
// and written to LDS in the layout of the direct-to-LDS tiles; W2 (converted to fp16 once
// per call) arrives by direct-to-LDS loads.  Tiles, waves and epilogue as gemm256_kernel;
// the MFMA is v_mfma_f32_32x32x16_f16.
// ---------------------------------------------------------------------------------
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
constexpr int kGateTableBytes = 2048 * 4;  // gamma | beta as fp16 pairs, K <= 2048

template <bool AFF>
__global__ __launch_bounds__(kBigThreads, 1) void gate_gemm_kernel(GateGemmArgs g) {
  constexpr int TM = 64, TN = 128;  // wave tile: tokens x features
  constexpr int MT = TM / 32, NT = TN / 32;
  constexpr int STAGE = kBigTile * kBigBK * 2;             // bytes of one operand stage
  constexpr int SEGS = STAGE / 1024 / (kBigThreads / 64);  // 1 KB W segments per wave
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  unsigned char *xs = smem;                        // G stages
  unsigned char *wsm = smem + kBigStages * STAGE;  // W stages
  // tables in arrays of their own, so that the compiler can tell them apart from the
  // direct-to-LDS writes in flight to the stages (and puts no load wait before reading them)
  __shared__ h2 gbt[kGateTableBytes / 4];          // gamma | beta, fp16
  __shared__ float2 rst[kBigTile];                 // (mean, 1 / std) of the tile's rows
  // an fp16 result that overflows clamps to +-65504 (G saturates instead of turning inf)
  __builtin_amdgcn_s_setreg((0 << 11) | (23 << 6) | 1, 1);

  const int N = g.N, K = g.K;
  // XCD-contiguous tile ranges over the tiles present (as gemm256_kernel)
  const int M = rows_present(g.m_dev, g.M);
  const int tiles = min(g.n_tiles_total, (M + kBigTile - 1) / kBigTile * g.n_tiles_n);
  const int per_xcd = (tiles + 7) / 8;
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int lin = xcd * per_xcd + slot;
  if (slot >= per_xcd || lin >= tiles) return;
  const int tile_n = lin % g.n_tiles_n;
  const int tile_m = lin / g.n_tiles_n;
  const int m0 = tile_m * kBigTile, n0 = tile_n * kBigTile;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 3, wn = wave >> 2;

  if constexpr (AFF) {
    for (int i = tid; i < K; i += kBigThreads) gbt[i] = h2{g.gb[i], g.gb[K + i]};
  }
  const __amdgpu_buffer_rsrc_t wr = uniform_rsrc(g.w + (int64_t)n0 * K, min(kBigTile, N - n0) * K * 2);
  const int lrow8 = lane / kCPR, lchunk = lane % kCPR;
  auto issue_w = [&](int kt) {
    const int stage = kt % kBigStages, k0 = kt * kBigBK;
#pragma unroll
    for (int j = 0; j < SEGS; ++j) {
      const int seg = j * 8 + wave;
      const int r = seg * (64 / kCPR) + lrow8;
      const int c = lchunk ^ ((r >> 1) & 7);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, wsm + stage * STAGE + seg * 1024, 16,
                                               (r * K + k0 + c * 8) * 2, 0, 0, 0);
    }
  };

  // Staging of G: wave w forms rows 32 w .. 32 w + 31 of the tile; lane l takes 16-byte
  // chunk l % 8 (8 features of one head, dv >= 32) of rows 32 w + l / 8 + 8 j, j = 0..3,
  // so that each load instruction reads 8 whole 128-byte row slices.
  const int gc = lane & 7;
  int grow_[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 32 * wave + (lane >> 3) + 8 * j;
    grow_[j] = m0 + r < M ? m0 + r : 0;
  }
  // the LayerNorm statistics (mean, 1 / std) of the tile's rows from the heads' (mean,
  // variance), into LDS (lanes 0..31 of wave w: row 32 w + lane)
  // (heads in groups of 8 loads issued together, the first group kept for the second
  // pass: a loop of one load per head, each waited for in turn, made 16 round trips per
  // tile before the first MFMA; indices past the last head read the last head again and
  // are left out of the sums after all 8 are issued)
  if (lane < 32) {
    const int r = m0 + 32 * wave + lane;
    const float2 *srow = g.stats + (int64_t)(r < M ? r : 0) * g.H;
    float2 st0[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) st0[i] = srow[min(i, g.H - 1)];
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m += i < g.H ? st0[i].x : 0.f;
    for (int h0 = 8; h0 < g.H; h0 += 8) {
      float2 st[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) st[i] = srow[min(h0 + i, g.H - 1)];
#pragma unroll
      for (int i = 0; i < 8; ++i) m += h0 + i < g.H ? st[i].x : 0.f;
    }
    m *= 1.0f / g.H;
    float v = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float d = st0[i].x - m;
      v += i < g.H ? st0[i].y + d * d : 0.f;
    }
    for (int h0 = 8; h0 < g.H; h0 += 8) {
      float2 st[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) st[i] = srow[min(h0 + i, g.H - 1)];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float d = st[i].x - m;
        v += h0 + i < g.H ? st[i].y + d * d : 0.f;
      }
    }
    v *= 1.0f / g.H;
    rst[32 * wave + lane] = float2{m, __builtin_amdgcn_rsqf(v + g.eps)};
  }

  u32x4 cv[4], uv[4];
  float2 hs[4];
  // c, U and the head statistics of chunk j of this lane for stage kt: exactly three load
  // instructions, issued by every lane, so that the waits in the k loop can count them.
  // Rows past M read row 0 and form rows of G that only reach output rows past M, which
  // are never stored; nothing selects on the loaded values, which would force a wait for
  // them right here.
  auto load_chunk = [&](int kt, int j) {
    const int f0 = kt * kBigBK + 8 * gc;
    const int64_t r = grow_[j];
    cv[j] = *reinterpret_cast<const u32x4 *>(g.c + r * K + f0);
    uv[j] = *reinterpret_cast<const u32x4 *>(g.u + r * g.u_stride + f0);
    hs[j] = g.stats[r * g.H + f0 / g.dv];
  };
  // G of chunk j of this lane for stage kt (registers -> LDS)
  float2 rsr[4];  // (mean, 1 / std) of the rows of this lane's chunks, read once
  auto store_chunk = [&](int kt, int j) {
    const int stage = kt % kBigStages, f0 = kt * kBigBK + 8 * gc;
    const int r = 32 * wave + (lane >> 3) + 8 * j;
    const float2 rs = rsr[j];
    const float a = __builtin_amdgcn_sqrtf(hs[j].y) * rs.y, b = (hs[j].x - rs.x) * rs.y;
    const h2 a2 = {(_Float16)a, (_Float16)a}, b2 = {(_Float16)b, (_Float16)b};
    // vector elements are copied to scalars before any bit cast: a bit cast taken
    // straight from a vector element is miscompiled by this compiler (only element 0
    // survives)
    uint32_t out[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t ce = cv[j][e], ue = uv[j][e];
      h2 t = __builtin_elementwise_fma(__builtin_bit_cast(h2, ce), a2, b2);
      if constexpr (AFF) {
        const h2 gb = gbt[f0 + 2 * e], gb1 = gbt[f0 + 2 * e + 1];
        t = __builtin_elementwise_fma(t, h2{gb[0], gb1[0]}, h2{gb[1], gb1[1]});
      }
      out[e] = __builtin_bit_cast(uint32_t, t * __builtin_bit_cast(h2, ue));
    }
    *reinterpret_cast<u32x4 *>(xs + stage * STAGE + swz(r, gc)) = u32x4{out[0], out[1], out[2], out[3]};
  };

  f32x16 acc[NT][MT];
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int j = 0; j < MT; ++j) acc[i][j] = f32x16{};

  // Pipeline: W of stage kt + 1 goes out by direct-to-LDS loads at the top of iteration kt;
  // chunk j of this lane's G of stage kt + 1 is formed after MFMA k-step j of stage kt,
  // from registers loaded one iteration earlier, and the registers are refilled at once
  // with the same chunk of stage kt + 2.  The loop body has no branch: past the last stage
  // the loads repeat the last stage and the G / W writes go to the free buffer, so the
  // wait counts below are exact.  Loads complete in order: the top of iteration kt waits
  // for W of stage kt while the 12 later loads of stage kt + 1 fly on.
  constexpr int NGL = 12;  // loads of one stage's four chunks
  const int nk = K / kBigBK;
#pragma unroll
  for (int j = 0; j < 4; ++j) load_chunk(0, j);
  issue_w(0);
  __syncthreads();  // the row statistics and the gamma / beta table
#pragma unroll
  for (int j = 0; j < 4; ++j) rsr[j] = rst[32 * wave + (lane >> 3) + 8 * j];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    store_chunk(0, j);
    load_chunk(min(1, nk - 1), j);
  }

  const int lrow = lane & 31, lk = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    wait_vmcnt<NGL>();
    __syncthreads();  // every wave's G of stage kt is in LDS; stage kt - 1 is free
    issue_w(min(kt + 1, nk - 1));
    const unsigned char *xst = xs + (kt % kBigStages) * STAGE;
    const unsigned char *wst = wsm + (kt % kBigStages) * STAGE;
#pragma unroll
    for (int ks = 0; ks < kBigBK / 16; ++ks) {
      // fragments of k-step ks; the G chunk formed meanwhile covers their LDS latency
      f16x8 wf[NT], xf[MT];
      const int c = ks * 2 + lk;
#pragma unroll
      for (int i = 0; i < NT; ++i)
        wf[i] = as_f16x8(*reinterpret_cast<const u32x4 *>(wst + swz(wn * TN + i * 32 + lrow, c)));
#pragma unroll
      for (int j = 0; j < MT; ++j)
        xf[j] = as_f16x8(*reinterpret_cast<const u32x4 *>(xst + swz(wm * TM + j * 32 + lrow, c)));
      // chunk ks of stage kt + 1 was loaded one iteration ago; 13 loads followed it (the
      // other chunks of its stage, W of stage kt + 1, this stage's refills before it)
      // nothing that uses chunk ks's registers may be scheduled above its wait
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<NGL + SEGS - 3>();
      store_chunk(kt + 1, ks);
      load_chunk(min(kt + 2, nk - 1), ks);
#pragma unroll
      for (int i = 0; i < NT; ++i)
#pragma unroll
        for (int j = 0; j < MT; ++j) acc[i][j] = mfma32_f16(wf[i], xf[j], acc[i][j]);
    }
  }
  wait_vmcnt<0>();  // the repeated last-stage loads land before LDS is reused below

  // epilogue through LDS, whole-row bf16 stores (as gemm256_kernel)
  __syncthreads();
#pragma unroll
  for (int j = 0; j < MT; ++j) {
    const int r = wm * TM + j * 32 + lrow;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = wn * TN + i * 32 + 8 * q + 4 * lk;
        float v0 = acc[i][j][4 * q + 0], v1 = acc[i][j][4 * q + 1];
        float v2 = acc[i][j][4 * q + 2], v3 = acc[i][j][4 * q + 3];
        if (g.bias != nullptr && n0 + c < N) {
          const f32x4 bb = *reinterpret_cast<const f32x4 *>(g.bias + n0 + c);
          v0 += bb[0]; v1 += bb[1]; v2 += bb[2]; v3 += bb[3];
        }
        *reinterpret_cast<u32x2 *>(smem + r * kOutPitch + c * 2) = u32x2{pack_bf16(v0, v1), pack_bf16(v2, v3)};
      }
    }
  }
  __syncthreads();
  constexpr int kRowChunks = kBigTile * 2 / 16;
#pragma unroll
  for (int it = 0; it < kBigTile * kRowChunks / kBigThreads; ++it) {
    const int ch = it * kBigThreads + tid;
    const int r = ch / kRowChunks, c16 = ch % kRowChunks;
    if (m0 + r < M && n0 + c16 * 8 < N) {
      const u32x4 v = *reinterpret_cast<const u32x4 *>(smem + r * kOutPitch + c16 * 16);
      *reinterpret_cast<u32x4 *>(g.out + (int64_t)(m0 + r) * N + n0 + c16 * 8) = v;
    }
  }
}

// The same product for rows of at most kGateTabHeads heads, with the per-head LayerNorm
// coefficients (a_h, b_h) of the tile's rows computed once per tile into an LDS table
// (fp16 pairs) instead of being loaded and derived per staged chunk.  That
// leaves two loads per chunk (c and U, by buffer loads whose stage and row group ride in the
// scalar offset, so the per-lane offsets are two registers), and the registers it frees
// double-buffer the operand fragments as in gemm256_kernel: the fragments of k-step ks + 1
// are read while the MFMAs of k-step ks run.  Rows past M read as zero (buffer range) and
// form zero rows of G, which only reach output rows that are not stored.  The arithmetic of
// a, b and G is that of gate_gemm_kernel, so both give the same bits.
constexpr int kGateTabHeads = 16;

template <bool AFF>
__global__ __launch_bounds__(kBigThreads, 1) void gate_gemm_tab_kernel(GateGemmArgs g) {
  constexpr int TM = 64, TN = 128;  // wave tile: tokens x features
  constexpr int MT = TM / 32, NT = TN / 32;
  constexpr int STAGE = kBigTile * kBigBK * 2;             // bytes of one operand stage
  constexpr int SEGS = STAGE / 1024 / (kBigThreads / 64);  // 1 KB W segments per wave
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  unsigned char *xs = smem;                        // G stages
  unsigned char *wsm = smem + kBigStages * STAGE;  // W stages
  __shared__ h2 gbt[kGateTableBytes / 4];              // gamma | beta, fp16
  // (a_h, b_h) fp16 of head h and tile row r = 32 w + l + 8 j (l < 8, j < 4) at
  // h 256 + 32 w + 4 l + j: the four rows a lane stages in one stage are one 16-byte read
  __shared__ __attribute__((aligned(16))) uint32_t abt[kGateTabHeads * kBigTile];
  // an fp16 result that overflows clamps to +-65504 (G saturates instead of turning inf)
  __builtin_amdgcn_s_setreg((0 << 11) | (23 << 6) | 1, 1);

  const int N = g.N, K = g.K, H = g.H;
  // XCD-contiguous tile ranges over the tiles present (as gemm256_kernel)
  const int M = rows_present(g.m_dev, g.M);
  const int tiles = min(g.n_tiles_total, (M + kBigTile - 1) / kBigTile * g.n_tiles_n);
  const int per_xcd = (tiles + 7) / 8;
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int lin = xcd * per_xcd + slot;
  if (slot >= per_xcd || lin >= tiles) return;
  const int tile_n = lin % g.n_tiles_n;
  const int tile_m = lin / g.n_tiles_n;
  const int m0 = tile_m * kBigTile, n0 = tile_n * kBigTile;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 3, wn = wave >> 2;
  const int rows = min(kBigTile, M - m0);

  // the heads' statistics of row 32 w + lane (lanes 0..31 of wave w), all loads issued at once
  float2 st[kGateTabHeads];
  if (lane < 32) {
    const int r = m0 + 32 * wave + lane;
    const float2 *srow = g.stats + (int64_t)(r < M ? r : 0) * H;
#pragma unroll
    for (int i = 0; i < kGateTabHeads; ++i) st[i] = srow[min(i, H - 1)];
  }

  const __amdgpu_buffer_rsrc_t wr = uniform_rsrc(g.w + (int64_t)n0 * K, min(kBigTile, N - n0) * K * 2);
  const int lrow8 = lane / kCPR, lchunk = lane % kCPR;
  auto issue_w = [&](int kt) {
    const int stage = kt % kBigStages, k0 = kt * kBigBK;
#pragma unroll
    for (int j = 0; j < SEGS; ++j) {
      const int seg = j * 8 + wave;
      const int r = seg * (64 / kCPR) + lrow8;
      const int c = lchunk ^ ((r >> 1) & 7);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, wsm + stage * STAGE + seg * 1024, 16,
                                               (r * K + k0 + c * 8) * 2, 0, 0, 0);
    }
  };

  // Staging of G: wave w forms rows 32 w .. 32 w + 31 of the tile; lane l takes 16-byte
  // chunk l % 8 (8 features of one head, dv >= 32) of rows 32 w + l / 8 + 8 j, j = 0..3.
  // The lane's offsets cover row 32 w + l / 8; row group j and the stage go in the scalar
  // offset.
  const int gc = lane & 7;
  const int grl = 32 * wave + (lane >> 3);
  const int ustride = (int)g.u_stride;
  const __amdgpu_buffer_rsrc_t cr = uniform_rsrc(g.c + (int64_t)m0 * K, rows * K * 2);
  const __amdgpu_buffer_rsrc_t ur = uniform_rsrc(g.u + (int64_t)m0 * g.u_stride, rows * ustride * 2);
  const int cvo = (grl * K + 8 * gc) * 2, uvo = (grl * ustride + 8 * gc) * 2;
  u32x4 cv[4], uv[4];
  // c and U of chunk j of this lane for stage kt: exactly two load instructions, issued by
  // every lane, so that the waits in the k loop can count them
  auto load_chunk = [&](int kt, int j) {
    const int so = kt * kBigBK * 2;
    cv[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(cr, cvo, so + j * 8 * K * 2, 0));
    uv[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ur, uvo, so + j * 8 * ustride * 2, 0));
  };
#pragma unroll
  for (int j = 0; j < 4; ++j) load_chunk(0, j);
  issue_w(0);

  if constexpr (AFF) {
    for (int i = tid; i < K; i += kBigThreads) gbt[i] = h2{g.gb[i], g.gb[K + i]};
  }
  // LayerNorm of the row from its heads' (mean, variance), then each head's (a_h, b_h)
  if (lane < 32) {
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < kGateTabHeads; ++i) m += i < H ? st[i].x : 0.f;
    m *= 1.0f / H;
    float v = 0.f;
#pragma unroll
    for (int i = 0; i < kGateTabHeads; ++i) {
      const float d = st[i].x - m;
      v += i < H ? st[i].y + d * d : 0.f;
    }
    v *= 1.0f / H;
    const float rstd = __builtin_amdgcn_rsqf(v + g.eps);
    const int slot = 32 * wave + 4 * (lane & 7) + (lane >> 3);  // row 32 w + lane
#pragma unroll
    for (int i = 0; i < kGateTabHeads; ++i)
      if (i < H) abt[i * kBigTile + slot] = pack_f16(__builtin_amdgcn_sqrtf(st[i].y) * rstd, (st[i].x - m) * rstd);
  }

  // (a, b) of this lane's four rows for the head of its chunk in a stage; hb, kmod: the
  // head of the stage's first feature and that feature's place in it (a stage's 64
  // features cross at most one head boundary, since dv is a multiple of 32)
  // (the stage past the last, whose G is formed and never read, clamps to the last head)
  auto read_ab = [&](int hb, int kmod) {
    const int h = min(hb + (kmod + 8 * gc >= g.dv ? 1 : 0), H - 1);
    return *reinterpret_cast<const u32x4 *>(abt + h * kBigTile + 32 * wave + 4 * (lane >> 3));
  };
  // G of chunk j of this lane for stage kt (registers -> LDS), ab: the row's (a, b)
  auto store_chunk = [&](int kt, int j, uint32_t abw) {
    const int stage = kt % kBigStages, f0 = kt * kBigBK + 8 * gc;
    const int r = grl + 8 * j;
    const h2 ab = __builtin_bit_cast(h2, abw);
    const h2 a2 = {ab[0], ab[0]}, b2 = {ab[1], ab[1]};
    uint32_t out[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t ce = cv[j][e], ue = uv[j][e];
      h2 t = __builtin_elementwise_fma(__builtin_bit_cast(h2, ce), a2, b2);
      if constexpr (AFF) {
        const h2 gb = gbt[f0 + 2 * e], gb1 = gbt[f0 + 2 * e + 1];
        t = __builtin_elementwise_fma(t, h2{gb[0], gb1[0]}, h2{gb[1], gb1[1]});
      }
      out[e] = __builtin_bit_cast(uint32_t, t * __builtin_bit_cast(h2, ue));
    }
    *reinterpret_cast<u32x4 *>(xs + stage * STAGE + swz(r, gc)) = u32x4{out[0], out[1], out[2], out[3]};
  };

  f32x16 acc[NT][MT];
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int j = 0; j < MT; ++j) acc[i][j] = f32x16{};

  // Pipeline as gate_gemm_kernel with two loads per chunk: W of stage kt + 1 goes out at the
  // top of iteration kt; chunk j of stage kt + 1 is formed after k-step j's fragment reads
  // of stage kt, from registers loaded one iteration earlier, and refilled at once with the
  // same chunk of stage kt + 2.  Past the last stage the loads repeat the last stage and the
  // G / W writes go to the free buffer, so the wait counts are exact.
  constexpr int NGL = 8;  // loads of one stage's four chunks
  const int nk = K / kBigBK;
  const int dv = g.dv;
  __syncthreads();  // the (a, b) and gamma / beta tables
  {
    const u32x4 ab0 = read_ab(0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      store_chunk(0, j, ab0[j]);
      load_chunk(min(1, nk - 1), j);
    }
  }
  // head and in-head offset of the first feature of stage 1
  int hb1 = kBigBK / dv, kmod1 = kBigBK - hb1 * dv;

  const int lrow = lane & 31, lk = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    wait_vmcnt<NGL>();
    __syncthreads();  // every wave's G of stage kt is in LDS; stage kt - 1 is free
    issue_w(min(kt + 1, nk - 1));
    const u32x4 ab1 = read_ab(hb1, kmod1);  // for the G of stage kt + 1
    const unsigned char *xst = xs + (kt % kBigStages) * STAGE;
    const unsigned char *wst = wsm + (kt % kBigStages) * STAGE;
    f16x8 wf[2][NT], xf[2][MT];
    auto read_frags = [&](int ks, int set) __attribute__((always_inline)) {
      const int c = ks * 2 + lk;
#pragma unroll
      for (int i = 0; i < NT; ++i)
        wf[set][i] = as_f16x8(*reinterpret_cast<const u32x4 *>(wst + swz(wn * TN + i * 32 + lrow, c)));
#pragma unroll
      for (int j = 0; j < MT; ++j)
        xf[set][j] = as_f16x8(*reinterpret_cast<const u32x4 *>(xst + swz(wm * TM + j * 32 + lrow, c)));
    };
    read_frags(0, 0);
#pragma unroll
    for (int ks = 0; ks < kBigBK / 16; ++ks) {
      if (ks + 1 < kBigBK / 16) read_frags(ks + 1, (ks + 1) & 1);
      // chunk ks of stage kt + 1 was loaded one iteration ago; 10 loads followed it (the
      // other chunks of its stage, W of stage kt + 1, this stage's refills before it);
      // nothing that uses chunk ks's registers may be scheduled above its wait
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<NGL + SEGS - 2>();
      store_chunk(kt + 1, ks, ab1[ks]);
      load_chunk(min(kt + 2, nk - 1), ks);
#pragma unroll
      for (int i = 0; i < NT; ++i)
#pragma unroll
        for (int j = 0; j < MT; ++j) acc[i][j] = mfma32_f16(wf[ks & 1][i], xf[ks & 1][j], acc[i][j]);
    }
    // the next stage's first feature
    kmod1 += kBigBK;
    while (kmod1 >= dv) {
      kmod1 -= dv;
      ++hb1;
    }
  }
  wait_vmcnt<0>();  // the repeated last-stage loads land before LDS is reused below

  // epilogue through LDS, whole-row bf16 stores (as gemm256_kernel)
  __syncthreads();
#pragma unroll
  for (int j = 0; j < MT; ++j) {
    const int r = wm * TM + j * 32 + lrow;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = wn * TN + i * 32 + 8 * q + 4 * lk;
        float v0 = acc[i][j][4 * q + 0], v1 = acc[i][j][4 * q + 1];
        float v2 = acc[i][j][4 * q + 2], v3 = acc[i][j][4 * q + 3];
        if (g.bias != nullptr && n0 + c < N) {
          const f32x4 bb = *reinterpret_cast<const f32x4 *>(g.bias + n0 + c);
          v0 += bb[0]; v1 += bb[1]; v2 += bb[2]; v3 += bb[3];
        }
        *reinterpret_cast<u32x2 *>(smem + r * kOutPitch + c * 2) = u32x2{pack_bf16(v0, v1), pack_bf16(v2, v3)};
      }
    }
  }
  __syncthreads();
  constexpr int kRowChunks = kBigTile * 2 / 16;
#pragma unroll
  for (int it = 0; it < kBigTile * kRowChunks / kBigThreads; ++it) {
    const int ch = it * kBigThreads + tid;
    const int r = ch / kRowChunks, c16 = ch % kRowChunks;
    if (m0 + r < M && n0 + c16 * 8 < N) {
      const u32x4 v = *reinterpret_cast<const u32x4 *>(smem + r * kOutPitch + c16 * 16);
      *reinterpret_cast<u32x4 *>(g.out + (int64_t)(m0 + r) * N + n0 + c16 * 8) = v;
    }
  }
}

// The f2 operand conversion as its own launch, one item per thread.
__global__ __launch_bounds__(256) void gate_prep_kernel(W2Prep q) {
  __builtin_amdgcn_s_setreg((0 << 11) | (23 << 6) | 1, 1);  // saturate, as the f2 kernel
  gate_prep_item(q, (int64_t)blockIdx.x * 256 + threadIdx.x);
}

}  // namespace

size_t gate_gemm_lds_bytes(int K) {
  (void)K;  // the tables are static arrays sized for the largest K
  const size_t stages = 2 * (size_t)kBigStages * kBigTile * kBigBK * 2;
  return std::max(stages, (size_t)kBigTile * kOutPitch);
}

hipError_t launch_gate_prep(const uint16_t *w2, int64_t n_w, const float *gamma, const float *beta,
                            int K, uint16_t *w2h, uint16_t *gb, hipStream_t stream) {
  W2Prep q;
  q.w2 = w2;
  q.n_w = n_w;
  q.gamma = gamma;
  q.beta = beta;
  q.K = K;
  q.w2h = w2h;
  q.gb = reinterpret_cast<_Float16 *>(gb);
  const int64_t work = gate_prep_work(q);
  gate_prep_kernel<<<dim3((unsigned)((work + 255) / 256)), 256, 0, stream>>>(q);
  return hipGetLastError();
}

hipError_t launch_gate_gemm(const GateGemmArgs &a, bool affine, hipStream_t stream) {
  if (a.M == 0) return hipSuccess;
  if (a.K % kBigBK != 0 || a.K > 2048 || a.N % 64 != 0 || a.dv < 32 || a.dv % 32 != 0 ||
      a.H <= 0 || a.N > kGemmMaxK)
    return hipErrorInvalidValue;
  GateGemmArgs g = a;
  g.n_tiles_n = (a.N + kBigTile - 1) / kBigTile;
  g.n_tiles_total = ((a.M + kBigTile - 1) / kBigTile) * g.n_tiles_n;
  const int grid = (g.n_tiles_total + 7) / 8 * 8;
  const size_t lds = gate_gemm_lds_bytes(a.K);
  // the attribute allows the largest table (K = 2048); each launch asks for what it needs
  // the table kernel for rows of at most kGateTabHeads heads, else per-chunk statistics
  const bool tab = a.H <= kGateTabHeads;
  static bool attr_set[2][2] = {{false, false}, {false, false}};
  const void *fn = tab ? (affine ? (const void *)gate_gemm_tab_kernel<true> : (const void *)gate_gemm_tab_kernel<false>)
                       : (affine ? (const void *)gate_gemm_kernel<true> : (const void *)gate_gemm_kernel<false>);
  if (!attr_set[tab][affine]) {
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)gate_gemm_lds_bytes(2048));  // fixed size
    if (e != hipSuccess) return e;
    attr_set[tab][affine] = true;
  }
  if (tab && affine)
    gate_gemm_tab_kernel<true><<<dim3(grid), dim3(kBigThreads), lds, stream>>>(g);
  else if (tab)
    gate_gemm_tab_kernel<false><<<dim3(grid), dim3(kBigThreads), lds, stream>>>(g);
  else if (affine)
    gate_gemm_kernel<true><<<dim3(grid), dim3(kBigThreads), lds, stream>>>(g);
  else
    gate_gemm_kernel<false><<<dim3(grid), dim3(kBigThreads), lds, stream>>>(g);
  return hipGetLastError();
}

hipError_t launch_gemm(const uint16_t *A, const uint16_t *W, const float *bias, uint16_t *out,
                       int M, int N, int K, Act act, OutType out_type, hipStream_t stream,
                       const int32_t *m_dev, const W2Prep *prep) {
  // the f2 operand conversion in its own launch, after the product
  auto prep_alone = [&](hipError_t e) {
    if (e != hipSuccess || prep == nullptr || prep->w2h == nullptr) return e;
    return launch_gate_prep(prep->w2, prep->n_w, prep->gamma, prep->beta, prep->K, prep->w2h,
                            reinterpret_cast<uint16_t *>(prep->gb), stream);
  };
  if (M == 0) return prep_alone(hipSuccess);
  if (K > kGemmMaxK) return hipErrorInvalidValue;  // 32-bit offsets within a 256-row panel
  const bool big = (N % kBigTile) == 0 && M >= kBigTile;
  const bool wide = (N % 128) == 0;
  GemmArgs a{};
  a.x = A;
  a.ldx = K;
  a.w = W;
  a.ldw = K;
  a.bias = bias;
  a.out = out;
  a.m_dev = m_dev;
  a.M = M;
  a.N = N;
  a.K = K;
  a.k_split = K;
  a.splits = 1;
  a.n_tiles_n = N / kBigTile;
  a.n_tiles_total = (M + kBigTile - 1) / kBigTile * a.n_tiles_n;
  if (act == ACT_SILU && out_type == OUT_F16) {
    if (big) {
      if (prep != nullptr) a.prep = *prep;
      return launch_big<KC, KC, ACT_SILU, OUT_F16>(a, stream);
    }
    return prep_alone(wide ? launch_tile<128, 128, ACT_SILU, OUT_F16>(A, W, bias, out, M, N, K, stream, m_dev)
                           : launch_tile<128, 64, ACT_SILU, OUT_F16>(A, W, bias, out, M, N, K, stream, m_dev));
  }
  if (act == ACT_NONE && out_type == OUT_F16) {  // pre-activations (the backward's recompute)
    if (big) return prep_alone(launch_big<KC, KC, ACT_NONE, OUT_F16>(a, stream));
    return prep_alone(wide ? launch_tile<128, 128, ACT_NONE, OUT_F16>(A, W, bias, out, M, N, K, stream, m_dev)
                           : launch_tile<128, 64, ACT_NONE, OUT_F16>(A, W, bias, out, M, N, K, stream, m_dev));
  }
  if (act == ACT_NONE && out_type == OUT_BF16) {
    if (big) return prep_alone(launch_big<KC, KC, ACT_NONE, OUT_BF16>(a, stream));
    return prep_alone(wide ? launch_tile<128, 128, ACT_NONE, OUT_BF16>(A, W, bias, out, M, N, K, stream, m_dev)
                           : launch_tile<128, 64, ACT_NONE, OUT_BF16>(A, W, bias, out, M, N, K, stream, m_dev));
  }
  return hipErrorInvalidValue;
}

// Splits of the reduction for C = X^T W over K = T tokens: enough (tile, split) units to
// fill the GPU twice over, each split a multiple of 64 rows and at least 512 rows long.
static int tn_k_split(int M, int N, int K) {
  const int tiles = ((M + kBigTile - 1) / kBigTile) * ((N + kBigTile - 1) / kBigTile);
  int splits = std::max(1, 512 / tiles);
  int ks = (K + splits - 1) / splits;
  ks = std::max(512, (ks + kBigBK - 1) / kBigBK * kBigBK);
  return ks;
}

size_t gemm_tn_partial_bytes(int M, int N, int K) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  const int ks = tn_k_split(M, N, K);
  const int splits = (K + ks - 1) / ks;
  return splits > 1 ? (size_t)splits * M * N * sizeof(float) : 0;
}

hipError_t launch_gemm_nn_f32(const uint16_t *X, int64_t ldx, const uint16_t *W, int64_t ldw,
                              float *out, int M, int N, int K, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  if (K <= 0 || K % kBigBK != 0 || N % 64 != 0 || ldx > kGemmMaxK || ldx < K || ldw < N ||
      (int64_t)K * ldw * 2 >= ((int64_t)1 << 31))
    return hipErrorInvalidValue;
  GemmArgs a{};
  a.x = X;
  a.ldx = ldx;
  a.w = W;
  a.ldw = ldw;
  a.out = out;
  a.M = M;
  a.N = N;
  a.K = K;
  a.k_split = K;
  a.splits = 1;
  a.n_tiles_n = (N + kBigTile - 1) / kBigTile;
  a.n_tiles_total = (M + kBigTile - 1) / kBigTile * a.n_tiles_n;
  return launch_big<KC, KR, ACT_NONE, OUT_F32>(a, stream);
}

hipError_t launch_gemm_tn_f32(const uint16_t *X, int64_t ldx, const uint16_t *W, int64_t ldw,
                              float *out, int M, int N, int K, float *partial, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  if (K <= 0 || N % 64 != 0 || M % 4 != 0 || ldx < M || ldw < N) return hipErrorInvalidValue;
  GemmArgs a{};
  a.x = X;
  a.ldx = ldx;
  a.w = W;
  a.ldw = ldw;
  a.M = M;
  a.N = N;
  a.K = K;
  a.k_split = tn_k_split(M, N, K);
  a.splits = (K + a.k_split - 1) / a.k_split;
  if ((int64_t)a.k_split * std::max(ldx, ldw) * 2 >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  if (a.splits > 1 && partial == nullptr) return hipErrorInvalidValue;
  a.out = a.splits > 1 ? (void *)partial : (void *)out;
  a.n_tiles_n = (N + kBigTile - 1) / kBigTile;
  a.n_tiles_total = (M + kBigTile - 1) / kBigTile * a.n_tiles_n;
  hipError_t e = launch_big<KR, KR, ACT_NONE, OUT_F32>(a, stream);
  if (e != hipSuccess || a.splits == 1) return e;
  const int64_t n = (int64_t)M * N;
  const int blocks = (int)std::min<int64_t>((n / 4 + 255) / 256, 4096);
  sum_splits_kernel<<<blocks, 256, 0, stream>>>(partial, a.splits, n, out);
  return hipGetLastError();
}

}  // namespace hstu
