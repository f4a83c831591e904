// Jagged pointwise aggregated attention of the HSTU layer, equation 2:
//     O_h[i] = sum_j SiLU(q_i . k_j + rab^{p,t}(i, j)) v_j
// ("Actions Speak Louder than Words" as retold on chenhuiyu.github.io, section
// "HSTU Layer 到底改了什么"; no softmax and no row normalisation, section
// "不对序列做 softmax"), over keys allowed by a causal or M-FALCON candidate mask, on
// jagged batches computed at their true lengths (section "另外三块拼图", item 1).
//
// gfx950 design
//  * One workgroup = 4 waves = 128 query rows of one (sequence, head), two workgroups per
//    CU; each wave owns 32 query rows whose Q fragments stay in registers for the whole
//    key loop.
//  * Keys stream through LDS in tiles of 64 rows, loaded straight from HBM into LDS
//    (buffer loads with the LDS destination, no register round trip) two tiles ahead of
//    their use, into rings of two or three stages.  Rows past a segment's end are outside
//    the buffer range and arrive as zeros.  K and V are stored row-major and unpadded,
//    with 16-byte chunks XOR-swizzled by row so the fragment reads are conflict free.
//  * Scores are computed transposed, S^T = K Q^T (v_mfma_f32_32x32x16_f16), so that each
//    lane's accumulator holds 16 keys of one query; after bias, SiLU and masking these
//    16 values are exactly the lane's B operand (8 keys per k-step) of O^T += V^T P^T,
//    with no trip through LDS.  The V^T operand comes from row-major V through the
//    transposing LDS read (ds_read_b64_tr_b16).  Q, K, V and A are fp16 operands (the
//    same MFMA rate as bf16 on gfx950, 3 more mantissa bits); accumulation and O stay
//    fp32.  Scores are carried scaled by -log2(e) so SiLU costs exp2, add, reciprocal
//    and multiply per element.
//  * The key loop is a pipeline over 32-key blocks: each step computes the scores of
//    block b+1, the weights of block b and the P.V product of block b-1, which are
//    independent.  Inside a step they are software-pipelined by hand: score MFMA i and
//    P.V MFMA i alternate, each with a share of the SiLU arithmetic beside it, and the
//    K / V fragments are read two MFMAs ahead; scheduling groups pin that issue order.
//  * Whether a batch has prefix (history) keys is a template parameter, so the plain
//    causal path carries no segment selection.
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
//  * Tiles are skipped from the jagged offsets and the mask: a workgroup never loads a
//    tile that lies wholly after its queries (causal) or away from them (candidate self
//    term), and a wave's blocks outside its own range add exactly zero.  Only blocks that
//    straddle the diagonal are masked per element; masked pairs contribute exactly 0.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace hstu {

namespace {

constexpr int kBN = kAttnBlockN;  // 64 keys per stage
constexpr int kMaxPos = 1024;
constexpr int kMaxTime = 64;
constexpr float kNegLog2e = -1.4426950408889634f;  // scores are carried as -log2(e) x
constexpr float kNegLn2 = -0.6931471805599453f;     // undoes that scale on the output
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit data format
constexpr int kModeFp16Ovfl = (0 << 11) | (23 << 6) | 1;  // hwreg(HW_REG_MODE, 23, 1)

enum BiasKind { BIAS_CONST = 0, BIAS_TWO = 1, BIAS_GENERAL = 2 };

// Buffer resource over `bytes` bytes at `base`: loads past the end return 0, so rows
// beyond a sequence's last key are zero without any branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, kRsrcWord3);
}

__device__ __forceinline__ int sgpr(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Load of a value that no thread writes while the kernel runs, through the constant
// address space: with a uniform address it becomes a scalar load.
template <class T>
__device__ __forceinline__ T ld_const(const T *ptr) {
  return *(const __attribute__((address_space(4))) T *)ptr;
}

// For thr >= 1, (max(0, ts_q - ts_k) >= thr) holds exactly when ts_k < key_limit(ts_q,
// thr) over the full int32 range: the difference is taken in 64 bits, and a limit below
// INT32_MIN (no key passes) clamps to INT32_MIN, which no int32 is below.
__device__ __forceinline__ int32_t key_limit(int32_t ts_q, uint32_t thr) {
  const int64_t lim = (int64_t)ts_q - (int64_t)thr + 1;
  return (int32_t)(lim < (int64_t)INT32_MIN ? (int64_t)INT32_MIN : lim);
}

// LDS tiles hold the CPR = DH / 8 chunks of 16 bytes of each key row, unpadded; chunk c
// of row r sits at chunk position c ^ swz(r), with RPS = 16 / CPR rows per 256-byte bank
// span:
//  * K: swz = (r / RPS) % CPR.  A score k-step reads one chunk of 32 consecutive rows;
//    any 16 of them then fall on 16 different 16-byte bank groups.
//  * V: swz = 4 ((r / RPS) % (4 / RPS)) (none for DH = 32).  A transposing read takes 4
//    consecutive rows x 4 chunks per half-wave, which then fall on disjoint bank groups.
// A stage is filled by 1 KB direct-to-LDS buffer loads (lane l writes bytes [16 l, 16 l +
// 16) of its KB); each lane loads the global chunk whose swizzled position that is.
template <int DH>
struct TileLayout {
  static constexpr int CPR = DH / 8;
  static constexpr int RPS = 16 / CPR;
  static constexpr int ROW = DH * 2;             // bytes per key row
  static constexpr int K_BYTES = kBN * ROW;
  static constexpr int V_BYTES = kBN * ROW;
  static constexpr int NI_K = K_BYTES / 1024;    // loads per K stage
  static constexpr int NI_V = V_BYTES / 1024;
  __device__ static int kswz(int r) { return (r / RPS) % CPR; }
  __device__ static int vswz(int r) { return 4 * ((r / RPS) % (4 / RPS)); }
};

// Scalar description of one 32-key block as seen by one wave, read from the wave's block
// table (three words) plus the block's index.
struct BlockInfo {
  uint32_t bits;  // bit 0 live: some key is visible to some query of the wave;
                  // bit 1 masked: the mask applies per element; bit 2 prefix (history) rows;
                  // bits 3-4 BiasKind; bits 5-10 the lower time bucket of the block
  int g;          // block index in the wave's key sequence (prefix blocks first)
  int l;          // lane of the block table that describes the block
  uint32_t c;     // CONST: the bias as the fp16 word of the bias MFMA operand
  __device__ bool live() const { return bits & 1u; }
  __device__ bool masked() const { return bits & 2u; }
  __device__ bool pre() const { return bits & 4u; }
  __device__ int kind() const { return (int)((bits >> 3) & 3u); }
  // TWO: keys whose gap reaches thr() (2^(lower bucket + 1) - 1) take hi
  __device__ uint32_t thr() const { return (uint32_t)(((uint64_t)1 << (((bits >> 5) & 63u) + 1)) - 1); }
};

template <int DH, int MASK, int NW, bool PRE>
__global__ __launch_bounds__(64 * NW, 2) void attn_kernel(AttnArgs p) {
  using L = TileLayout<DH>;
  constexpr int NT = 64 * NW;          // threads per workgroup
  constexpr int BM = 32 * NW;          // query rows per workgroup
  constexpr int KS = DH / 16;          // k-steps of the score MFMA
  constexpr int FT = DH / 32;          // 32-wide feature tiles of the output
  // Loads of one batch: the K KBs of a tile and the V KBs of a tile, LPW per wave (load j
  // of a wave is KB number wave + NW j, K first), and the tile's key timestamps (wave 0).
  // A batch thus adds LPW to the vector-memory count of every wave but wave 0 (LPW + 1),
  // and the barrier's count wait (sized for LPW) holds wave 0 slightly longer than needed.
  constexpr int NL = L::NI_K + L::NI_V;
  static_assert(NL % NW == 0, "whole loads per wave");
  constexpr int LPW = NL / NW;
  constexpr bool K_FIXED = L::NI_K % NW == 0;  // load j's kind is the same in every wave
  // Stages per ring and how many tiles ahead the loads run: three stages (two tiles of
  // lead) where LDS allows it, two for the 4-wave groups at DH = 128, which then fit two
  // workgroups per CU.
  constexpr int NS = (NW == 8 || DH <= 64) ? 3 : 2;
  constexpr int LEAD = NS - 1;

  // K and V stages, each its own LDS array: every access names its array at compile time
  // (the tile loop is unrolled by NS), so the compiler can tell that a read of one stage
  // does not alias the direct-to-LDS writes in flight to another and puts no
  // vector-memory wait before it.  It tells apart only a few such destinations, so the
  // tile's key timestamps ride at the end of its K stage (2 NS arrays in all).
  constexpr int KT_BYTES = L::K_BYTES + kBN * 4;
  __shared__ __attribute__((aligned(16))) unsigned char k_st0[KT_BYTES], k_st1[KT_BYTES], k_st2[KT_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char v_st0[L::V_BYTES], v_st1[L::V_BYTES], v_st2[L::V_BYTES];
  auto kbuf = [&](auto s_c) __attribute__((always_inline)) -> unsigned char * {
    constexpr int S = decltype(s_c)::value;
    if constexpr (S == 0) return k_st0;
    else if constexpr (S == 1) return k_st1;
    else return k_st2;
  };
  auto vbuf = [&](auto s_c) __attribute__((always_inline)) -> unsigned char * {
    constexpr int S = decltype(s_c)::value;
    if constexpr (S == 0) return v_st0;
    else if constexpr (S == 1) return v_st1;
    else return v_st2;
  };
  auto tbuf = [&](auto s_c) __attribute__((always_inline)) -> int32_t * {
    return reinterpret_cast<int32_t *>(kbuf(s_c) + L::K_BYTES);
  };
  __shared__ float ptab[kMaxPos];
  __shared__ float ttab[kMaxTime];

  // workgroup b takes work item b / H for head b % H: every head's longest items start
  // first (head-major order, through the grid's y, started the last head's longest items
  // only near the end of the launch: 3% longer inside the stack)
  const int item = (int)blockIdx.x / p.num_heads;
  if (item >= ld_const(p.n_work)) return;
  uint64_t clk0 = 0, rt0 = 0;  // lifetime clocks, when profiling
  if (p.clk != nullptr) {
    clk0 = __builtin_amdgcn_s_memtime();
    rt0 = __builtin_amdgcn_s_memrealtime();
  }
  // MODE.FP16_OVFL: an fp16 result that overflows clamps to +-65504 instead of becoming
  // infinite.  The weights A are packed to fp16 in the scaled domain (A / -ln 2), so a
  // score whose SiLU exceeds 65504 ln 2 (about 45403) contributes that value instead of
  // turning the row infinite, at no cost per element.
  __builtin_amdgcn_s_setreg(kModeFp16Ovfl, 1);
  const int h = (int)blockIdx.x % p.num_heads;
  const int b = ld_const(p.work + 2 * item), qt = ld_const(p.work + 2 * item + 1);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = sgpr(tid >> 6);
  const int lrow = lane & 31, half = lane >> 5;

  const int s0 = ld_const(p.offsets + b);
  const int n = ld_const(p.offsets + b + 1) - s0;
  const int q0 = qt * BM;
  constexpr bool has_prefix = PRE;
  const int p0 = has_prefix ? ld_const(p.p_offsets + b) : 0;
  const int n_p = has_prefix ? ld_const(p.p_offsets + b + 1) - p0 : 0;
  const bool use_pos = p.rab_pos != nullptr;
  const bool use_time = p.rab_time != nullptr && p.ts != nullptr &&
                        (!PRE || p.p_ts != nullptr);
  const int rrow = p.rab_per_head ? h : 0;

  // Scores are carried scaled by -log2(e): t = -log2(e) (q.k + bias), so that
  // SiLU(x) = x / (1 + e^-x) = -ln(2) t / (1 + 2^t).  Q and the bias tables are scaled
  // once here, each score element costs exp2, add, reciprocal and multiply, and the
  // factor -ln(2) is applied to the output accumulators once, at the end.
  // Prologue.  Every global read that the key loop depends on goes out before any of them
  // is waited for: the bias tables, the queries' timestamps, Q, the key timestamp ranges
  // of the first block table, then the first K / V batches.  They are consumed in that
  // order, so the prologue costs one memory round trip instead of one per step, and the
  // K / V batches stay in flight through the rest of it.
  // relative-bias tables of this head (into LDS, scaled, below)
  constexpr int PJ = (kMaxPos + NT - 1) / NT;
  static_assert(kMaxTime <= NT, "one time bucket per thread");
  float pv[PJ], tv = 0.0f;
  if (use_pos) {
#pragma unroll
    for (int j = 0; j < PJ; ++j)
      if (j * NT < p.pos_buckets) pv[j] = p.rab_pos[rrow * p.pos_buckets + min(tid + j * NT, p.pos_buckets - 1)];
  }
  {  // no branch around the load (a branch drew the scaling, and so a wait, up to it);
     // without the time term the range is empty and the load reads zero
    const __amdgpu_buffer_rsrc_t rtt =
        make_rsrc(use_time ? p.rab_time + rrow * p.time_buckets : nullptr, use_time ? p.time_buckets * 4u : 0u);
    tv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rtt, min(tid, kMaxTime - 1) * 4, 0, 0));
  }

  // this wave's queries: local index qi, position, timestamp; Q fragments in registers
  const int qbase = q0 + wave * 32;  // wave-uniform
  const int qi = qbase + lrow;
  const bool q_ok = qi < n;
  const bool wave_has_rows = qbase < n;
  const int qpos = MASK == 0 ? n_p + qi : n_p;
  const int32_t qts = use_time ? p.ts[s0 + (q_ok ? qi : n - 1)] : 0;
  const int qpos_min = MASK == 0 ? n_p + qbase : n_p;
  const int qmax = qbase + 31;
  // Q rows of this head through a descriptor over the sequence's rows: rows past its end
  // read as zero, with no branch around the loads
  u32x4 qraw[KS];
  {
    const __amdgpu_buffer_rsrc_t rq =
        make_rsrc(p.q + (int64_t)s0 * p.stride + h * DH, (uint32_t)n * (uint32_t)p.stride * 2u);
    const int qoff = (qi * (int)p.stride + half * 8) * 2;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qraw[ks] = __builtin_amdgcn_raw_buffer_load_b128(rq, qoff + ks * 32, 0, 0);
  }
  // A operand of one extra k-step that adds a per-block constant to every score: 1 at
  // k = 0 for every key row (lanes 0-31 hold k = 0..7), 0 elsewhere.  Its B operand holds
  // the constant (fp16) at k = 0, so a constant-bias block starts its score chain with
  // one MFMA on a zero accumulator instead of 16 register moves per lane.
  const f16x8 kf_one = as_f16x8(u32x4{half == 0 ? 0x3C00u : 0u, 0u, 0u, 0u});

  // key tiles: prefix tiles first, then own tiles
  const int n_pt = (n_p + kBN - 1) / kBN;
  const int q_end = min(n, q0 + BM);
  const int own_start = MASK == 0 ? 0 : q0;
  const int n_ot = (q_end - own_start + kBN - 1) / kBN;
  const int n_tiles = n_pt + n_ot;

  // Byte offset, within the tile's rows of pitch rowb bytes, of the global chunk that this
  // lane's element of load j (KB number id = w + NW j) brings to its swizzled position.
  auto load_off = [&](int j, uint32_t rowb_, int w) __attribute__((always_inline)) {
    const int id = w + NW * j;
    const bool is_k = id < L::NI_K;
    const int pos = (is_k ? id : id - L::NI_K) * 64 + lane;  // chunk position in the stage
    const int r = pos / L::CPR;
    const int c = (pos % L::CPR) ^ (is_k ? L::kswz(r) : L::vswz(r));
    return r * (int)rowb_ + c * 16;
  };
  // The offsets stay in registers that are used for nothing else: the compiler treats the
  // offset register of a direct-to-LDS load as busy until the load completes, so a copy
  // that it later reused would stall on the load.  Prefix and own rows share one pitch
  // (the entry point checks it).
  const uint32_t rowb = (uint32_t)p.stride * 2;
  int ld_off[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) ld_off[j] = load_off(j, rowb, wave);
  const int ts_off = lane * 4;

  auto seg_of = [&](int t, int &kbase, int &limit) __attribute__((always_inline)) {
    const bool pre = PRE && t < n_pt;
    kbase = pre ? t * kBN : own_start + (t - n_pt) * kBN;
    limit = n + (pre ? n_p - n : 0);  // arithmetic, not a select between the captured variables
    return pre;
  };

  // Rows of this head in the two key segments: the prefix (history) rows of the sequence
  // and its own rows.  A tile's loads take a descriptor whose range is its whole segment
  // and reach the tile through the scalar offset, which the hardware range check includes:
  // rows past the segment's end arrive as zeros, and a tile outside [0, n_tiles) gets an
  // empty range.  Per tile this is a few scalar selects and one multiply.
  const int64_t stride = p.stride;
  const uint16_t *const k_own = p.k + (int64_t)s0 * stride + h * DH;
  const uint16_t *const v_own = p.v + (int64_t)s0 * stride + h * DH;
  const uint16_t *const k_pre = has_prefix ? p.pk + (int64_t)p0 * stride + h * DH : k_own;
  const uint16_t *const v_pre = has_prefix ? p.pv + (int64_t)p0 * stride + h * DH : v_own;
  const int32_t *const ts_own = use_time ? p.ts + s0 : p.offsets;
  const int32_t *const ts_pre = use_time && has_prefix ? p.p_ts + p0 : ts_own;
  // Segment (pre), first row (kbase) and row count of tile t; false if t is no tile.
  auto tile_seg = [&](int t, bool &pre, int &kbase, int &rows) __attribute__((always_inline)) {
    const bool valid = t >= 0 && t < n_tiles;
    int limit;
    pre = seg_of(valid ? t : 0, kbase, limit);
    rows = valid ? limit : 0;
    return valid;
  };
  // One batch: K rows and key timestamps of tile tk into K stage kstage_c, V rows of tile
  // tv into V stage vstage_c.  Part 0 issues the first half of the wave's loads (and the
  // timestamps), part 1 the second half, part 2 all of them: the iteration issues the two
  // halves at two points, so that the four waves of a workgroup do not queue all their
  // loads on the CU's vector-memory path at the same moment.
  auto issue_batch = [&](int tk, int tv, auto kstage_c, auto vstage_c, auto part_c) __attribute__((always_inline)) {
    constexpr int PART = decltype(part_c)::value;
    constexpr int J0 = PART == 1 ? LPW / 2 : 0, J1 = PART == 0 ? LPW / 2 : LPW;
    bool pk_, pv_;
    int kb_k, kb_v, rows_k, rows_v;
    tile_seg(tk, pk_, kb_k, rows_k);
    tile_seg(tv, pv_, kb_v, rows_v);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(pk_ ? k_pre : k_own, (uint32_t)rows_k * rowb);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(pv_ ? v_pre : v_own, (uint32_t)rows_v * rowb);
    const int so_k = kb_k * (int)rowb, so_v = kb_v * (int)rowb;
#pragma unroll
    for (int j = J0; j < J1; ++j) {
      const int id = wave + NW * j;
      const bool is_k = K_FIXED ? j < L::NI_K / NW : id < L::NI_K;
      if (is_k) {
        unsigned char *lds = kbuf(kstage_c) + id * 1024;
        const int vo = ld_off[j];  // a local: an array element here loses the kernel's host stub
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, lds, 16, vo, so_k, 0, 0);
      } else {
        unsigned char *lds = vbuf(vstage_c) + (id - L::NI_K) * 1024;
        const int vo = ld_off[j];
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, lds, 16, vo, so_v, 0, 0);
      }
    }
    if (PART != 1 && wave == 0) {
      const uint32_t bytes = use_time ? (uint32_t)rows_k * 4u : 0u;
      const int so_t = kb_k * 4;
      unsigned char *lds = reinterpret_cast<unsigned char *>(tbuf(kstage_c));
      const __amdgpu_buffer_rsrc_t rt = make_rsrc(pk_ ? ts_pre : ts_own, bytes);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rt, lds, 4, ts_off, so_t, 0, 0);
    }
  };

  // Block table.  Block g of the wave's key sequence covers keys 32 (g mod 2) .. + 31 of
  // tile g / 2.  Lane i of the table describes block cbase + i: every lane classifies its
  // block in vector code, from the wave's query position / timestamp range and the
  // block's key timestamp range (precomputed by block_stats_kernel), once per 64 blocks;
  // the key loop then reads a block's entry with three v_readlane.  Classes:
  //   - live: some key is visible to some query of the wave; masked: the mask applies per
  //     element (the block straddles the diagonal, or the candidate self term);
  //   - bias kind: CONST when every relative position is past the last position bucket and
  //     the smallest and largest gap share one time bucket (the bucket being monotone in
  //     the gap); TWO when the gaps span exactly buckets b and b + 1; GENERAL otherwise.
  // A table is built in two parts: the block's geometry and the load of its key timestamp
  // range, then (once that has landed) the classification.
  int tab_bits = 0, tab_lo = 0, tab_hi = 0, tab_c = 0;
  int cbase = 0;
  struct TabLoad {
    int2 r;
    int k0;
    bool lv, mk, pre;
  };
  auto table_load = [&](int c0) __attribute__((always_inline)) {
    TabLoad tl;
    const int g = c0 + lane;
    const int t = g >> 1;
    const bool valid = t < n_tiles;
    tl.pre = PRE && t < n_pt;
    const int kbase = tl.pre ? t * kBN : own_start + (t - n_pt) * kBN;
    const int limit = n + (tl.pre ? n_p - n : 0);
    tl.k0 = kbase + (g & 1) * 32;
    tl.lv = valid && tl.k0 < limit && wave_has_rows;
    if (MASK == 0) {
      tl.lv = tl.lv && (tl.pre || tl.k0 <= qmax);
      tl.mk = !tl.pre && tl.k0 + 31 > qbase;
    } else {
      tl.lv = tl.lv && (tl.pre || (tl.k0 <= qmax && tl.k0 + 31 >= qbase));
      tl.mk = !tl.pre;
    }
    tl.r = int2{0, 0};
    if (use_time && tl.lv) tl.r = tl.pre ? p.p_kstat[p0 + tl.k0] : p.kstat[s0 + tl.k0];
    return tl;
  };
  // Batch b (issued in iteration b, or before the loop for b < -1) loads K of tile
  // b + 1 + LEAD into K stage (b mod NS) and V of tile b + LEAD into V stage
  // ((b - 1) mod NS): the stages that iteration b - 1 finished reading.  Iteration t
  // reads K of tile t + 1 and V of tile t, which batch t - LEAD brought; its barrier
  // waits for that batch and leaves the LEAD - 1 newer batches in flight.
  auto batch = [&](int b, auto r_c, auto part_c) __attribute__((always_inline)) {  // r_c = b mod NS
    constexpr int R = decltype(r_c)::value;
    issue_batch(b + 1 + LEAD, b + LEAD, std::integral_constant<int, R>{},
                std::integral_constant<int, (R + NS - 1) % NS>{}, part_c);
  };
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  using CLast = std::integral_constant<int, NS - 1>;
  // the first table's loads, then the first K / V batches (the last prologue loads)
  const TabLoad tl0 = table_load(0);
  if constexpr (NS == 3) {
    batch(-3, C0{}, std::integral_constant<int, 2>{});
    batch(-2, C1{}, std::integral_constant<int, 2>{});
  } else {
    batch(-2, C0{}, std::integral_constant<int, 2>{});
  }

  // the bias tables into LDS, scaled; the writes made visible to the workgroup without
  // waiting for the K / V batches (lgkmcnt(0) only, then a bare barrier)
  if (use_pos) {
#pragma unroll
    for (int j = 0; j < PJ; ++j)
      if (j * NT < p.pos_buckets && tid + j * NT < p.pos_buckets) ptab[tid + j * NT] = kNegLog2e * pv[j];
  }
  if (use_time && tid < p.time_buckets) ttab[tid] = kNegLog2e * tv;
  __builtin_amdgcn_s_waitcnt((3 << 14) | (7 << 4) | 15);  // lgkmcnt(0), vmcnt / expcnt not waited
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  // bias of every relative position past the last bucket
  const float pos_last = use_pos ? __builtin_bit_cast(float, sgpr(__builtin_bit_cast(int, ptab[p.pos_buckets - 1]))) : 0.0f;
  // timestamp range of the wave's queries, wave-uniform on every path
  int32_t qmn = q_ok ? qts : INT32_MAX, qmx = q_ok ? qts : INT32_MIN;
  if (use_time) {
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) {
      qmn = min(qmn, __shfl_xor(qmn, o, 64));
      qmx = max(qmx, __shfl_xor(qmx, o, 64));
    }
  }
  const int32_t qts_min = sgpr(qmn), qts_max = sgpr(qmx);
  // Q fragments, scaled by -log2(e)
  f16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const f16x8 raw = as_f16x8(qraw[ks]);
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = kNegLog2e * (float)raw[e];
    const u32x4 sc = {pack_f16(x[0], x[1]), pack_f16(x[2], x[3]),
                      pack_f16(x[4], x[5]), pack_f16(x[6], x[7])};
    qf[ks] = as_f16x8(sc);
  }
  // Complete the Q loads here, on every path: otherwise the wait-count pass can see them
  // as possibly in flight inside the key loop and drain all vector loads there, which
  // would also wait for the tile prefetch.  The empty asm only names the registers.
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) asm("" : "+v"(qf[ks]));

  // The bias of a block on the constant or two-bucket path is pos_last plus one entry of
  // the time table: lane i of tsum holds that sum for bucket i (at most 64 buckets).
  float tsum = pos_last;
  if (use_time && lane < p.time_buckets) tsum += ttab[lane];
  auto table_fin = [&](int c0, const TabLoad &tl) __attribute__((always_inline)) {
    const int kpos_max = tl.pre ? tl.k0 + 31 : (MASK == 0 ? n_p + tl.k0 + 31 : n_p);
    const bool pos_general = use_pos && qpos_min - kpos_max < p.pos_buckets - 1;
    int tb_lo = 0, tb_hi = 0;
    if (use_time) {
      tb_lo = min(time_log2_bucket(qts_min, tl.r.y), p.time_buckets - 1);
      tb_hi = min(time_log2_bucket(qts_max, tl.r.x), p.time_buckets - 1);
    }
    const int kind = pos_general || tb_hi > tb_lo + 1 ? BIAS_GENERAL : (tb_hi == tb_lo ? BIAS_CONST : BIAS_TWO);
    tab_bits = (tl.lv ? 1 : 0) | (tl.mk ? 2 : 0) | (tl.pre ? 4 : 0) | (kind << 3) | (tb_lo << 5);
    tab_lo = __builtin_bit_cast(int, __shfl(tsum, tb_lo, 64));
    tab_hi = __builtin_bit_cast(int, __shfl(tsum, tb_hi, 64));
    tab_c = (int)pack_f16(__builtin_bit_cast(float, tab_lo), 0.0f);  // CONST bias as the MFMA word
    cbase = c0;
  };
  auto build_table = [&](int c0) __attribute__((always_inline)) { table_fin(c0, table_load(c0)); };
  table_fin(0, tl0);
  auto fetch = [&](int g) __attribute__((always_inline)) {
    const int l = g - cbase;
    BlockInfo bi;
    bi.bits = (uint32_t)__builtin_amdgcn_readlane(tab_bits, l);
    bi.c = (uint32_t)__builtin_amdgcn_readlane(tab_c, l);
    bi.l = l;
    bi.g = g;
    return bi;
  };
  // first key index of a block within its segment
  const int own_k0_shift = own_start - n_pt * kBN;
  auto k0_of = [&](const BlockInfo &bi) __attribute__((always_inline)) {
    return bi.g * 32 + ((PRE && bi.pre()) ? 0 : own_k0_shift);
  };

  f32x16 acc_o[FT];
#pragma unroll
  for (int f = 0; f < FT; ++f) acc_o[f] = f32x16{};
  // B operand of the constant-bias MFMA: the bias word (k = 0) and three zero words
  u32x4 bq = {0u, 0u, 0u, 0u};

  // ---- the three parts of a step ----
  // Score accumulator init with the block's bias (CONST / TWO / GENERAL), from the key
  // timestamps tsb of the K stage.  s^T lane layout: query lrow, keys 8 (i / 4) + 4 half + i % 4.
  auto s_init = [&](f32x16 &s, const BlockInfo &bi, const int32_t *tsb, int blk, auto kind_c) __attribute__((always_inline)) {
    constexpr int KIND = decltype(kind_c)::value;
    const int32_t *kts = tsb + blk * 32 + 4 * half;
    if constexpr (KIND == BIAS_CONST) {
      bq.x = bi.c;
      s = mfma32_f16(kf_one, as_f16x8(bq), f32x16{});
    } else if constexpr (KIND == BIAS_TWO) {
      const int32_t klim = key_limit(qts, bi.thr());
      const float hi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(tab_hi, bi.l));
      const float lo = __builtin_bit_cast(float, __builtin_amdgcn_readlane(tab_lo, bi.l));
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int4 t4 = *reinterpret_cast<const int4 *>(kts + 8 * g);
        s[4 * g + 0] = t4.x < klim ? hi : lo;
        s[4 * g + 1] = t4.y < klim ? hi : lo;
        s[4 * g + 2] = t4.z < klim ? hi : lo;
        s[4 * g + 3] = t4.w < klim ? hi : lo;
      }
    } else {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        int4 t4 = {0, 0, 0, 0};
        if (use_time) t4 = *reinterpret_cast<const int4 *>(kts + 8 * g);
        const int32_t kt4[4] = {t4.x, t4.y, t4.z, t4.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float x = 0.0f;
          if (use_pos) {
            const int kidx = k0_of(bi) + 8 * g + 4 * half + r;
            const int kpos = (PRE && bi.pre()) ? kidx : (MASK == 0 ? n_p + kidx : n_p);
            x += ptab[min(max(qpos - kpos, 0), p.pos_buckets - 1)];
          }
          if (use_time) x += ttab[min(time_log2_bucket(qts, kt4[r]), p.time_buckets - 1)];
          s[4 * g + r] = x;
        }
      }
    }
  };
  // K fragment of score k-step ks: row lrow of the block, logical chunk 2 ks + half at its
  // swizzled position; the swizzle of row blk 32 + lrow is that of lrow, and it only flips
  // bits below the row pitch, so the address of k-step ks is k_base ^ (32 ks).
  const int k_base = lrow * L::ROW + ((half ^ L::kswz(lrow)) * 16);
  // O^T += V^T P^T over the block's 32 keys (V stage vs_buf).  The V^T operand comes from
  // row-major V through transposing reads: in each 16-lane group, lane 4 j + q names row
  // (key) kb + j at features 4 q .. 4 q + 3 of its 16-feature slice, and lane i receives
  // keys kb .. kb + 3 of feature i.  Two reads (keys +0 and +8) give the 8 keys of a
  // lane's k-step in the order of the P^T operand: key 16 s2 + 8 (e / 4) + 4 half + e % 4.
  // Lane: row 4 half + j (j = (lane % 16) / 4) of each 8-row group, logical chunk
  // 4 f + 2 ((lane / 16) % 2) + (lane % 4) / 2 of feature tile f, half (lane % 2) of the
  // chunk; the swizzle depends only on that row and flips bits below the row pitch, so the
  // address for feature tile f is v_base ^ (64 f).
  int v_base;
  {
    const int vr = (lane >> 5) * 4 + ((lane & 15) >> 2);
    v_base = vr * L::ROW + (((((lane >> 4) & 1) * 2 + ((lane & 3) >> 1)) ^ L::vswz(vr)) * 16) +
             (lane & 1) * 8;
  }
  // The step's three independent parts as one software pipeline of KS iterations:
  // iteration i issues score MFMA i (S^T += K Q^T, k-step i), P.V MFMA i (k-step i / FT,
  // feature tile i % FT) and the SiLU of 16 / KS score elements of the cur block, with
  // the K and V fragments read two iterations ahead.  The scheduling groups below keep
  // that order, so that consecutive MFMAs are independent, each has VALU work beside it,
  // and no MFMA waits on a fragment read.
  auto fused = [&](f32x16 &s, const unsigned char *ks_buf, int nblk, const f32x16 &sc,
                   f16x8 (&pc)[2], const f16x8 (&pp)[2], const unsigned char *vs_buf,
                   int pblk) __attribute__((always_inline)) {
    const unsigned char *kb = ks_buf + nblk * 32 * L::ROW;
    const unsigned char *vb = vs_buf + pblk * 32 * L::ROW;
    constexpr int EPI = 16 / KS;  // SiLU elements per iteration
    f16x8 kf[KS], vf[KS];
    auto rk = [&](int i) __attribute__((always_inline)) {
      kf[i] = as_f16x8(*reinterpret_cast<const u32x4 *>(kb + (k_base ^ (i * 32))));
    };
    auto rv = [&](int i) __attribute__((always_inline)) {
      const int s2 = i / FT, f = i % FT;
      const u32x2 lo = lds_read_tr16(vb + (16 * s2) * L::ROW + (v_base ^ (64 * f)));
      const u32x2 hi = lds_read_tr16(vb + (16 * s2 + 8) * L::ROW + (v_base ^ (64 * f)));
      vf[i] = as_f16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
    };
    float a[16];
    rk(0);
    rv(0);
    if constexpr (KS > 1) {
      rk(1);
      rv(1);
    }
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      if (i + 2 < KS) {
        rk(i + 2);
        rv(i + 2);
      }
      s = mfma32_f16(kf[i], qf[i], s);
#pragma unroll
      for (int e = EPI * i; e < EPI * (i + 1); ++e) {
        const float t = sc[e];
        a[e] = t * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(t));
      }
      acc_o[i % FT] = mfma32_f16(vf[i], pp[i / FT], acc_o[i % FT]);
    }
    pc[0] = as_f16x8(u32x4{pack_f16(a[0], a[1]), pack_f16(a[2], a[3]), pack_f16(a[4], a[5]),
                           pack_f16(a[6], a[7])});
    pc[1] = as_f16x8(u32x4{pack_f16(a[8], a[9]), pack_f16(a[10], a[11]), pack_f16(a[12], a[13]),
                           pack_f16(a[14], a[15])});
    // issue order: 6 fragment reads, then per iteration score MFMA, 3 reads, half of the
    // SiLU work, P.V MFMA, the other half
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // score MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);          // fragment reads
      __builtin_amdgcn_sched_group_barrier(0x400, EPI, 0);        // exp
      __builtin_amdgcn_sched_group_barrier(0x002, EPI, 0);        // add
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // P.V MFMA
      __builtin_amdgcn_sched_group_barrier(0x400, EPI, 0);        // rcp
      __builtin_amdgcn_sched_group_barrier(0x002, EPI + EPI / 2, 0);  // mul, pack
    }
  };

  using KConst = std::integral_constant<int, BIAS_CONST>;
  using KTwo = std::integral_constant<int, BIAS_TWO>;
  using KGen = std::integral_constant<int, BIAS_GENERAL>;

  // Scores of a block that must not contribute (masked elements; every element of a block
  // outside the wave's range) are set to +1e30, a very negative score in the scaled domain:
  // the weight is then exactly zero (2^t overflows to +inf, its reciprocal is 0, and
  // 1e30 * 0 = 0).
  auto mask_scores = [&](f32x16 &s, const BlockInfo &bi) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kidx = k0_of(bi) + 8 * (i >> 2) + 4 * half + (i & 3);
      const bool allowed = bi.live() && (!bi.masked() || (MASK == 0 ? kidx <= qi : kidx == qi));
      s[i] = allowed ? s[i] : 1e30f;
    }
  };

  // One step of the block pipeline: S of block "next", SiLU of block "cur", P.V of block
  // "prev".  The three parts are independent and always run as one straight-line basic
  // block (a block outside the wave's range costs its MFMAs but adds exactly zero), so
  // the compiler overlaps the SiLU arithmetic with the MFMAs and the output accumulators
  // are updated in one place only.  Only the score initialisation branches on the bias
  // kind, and a step with all three blocks outside the range only clears the cur block's P.
  auto step = [&](f32x16 &s_next, const BlockInfo &bn, const unsigned char *kst, const int32_t *tst,
                  int nblk, f32x16 &s_cur, f16x8 (&p_cur)[2], const BlockInfo &bc,
                  const f16x8 (&p_prev)[2], const BlockInfo &bp, const unsigned char *vst, int pblk) __attribute__((always_inline)) {
    if (!bn.live() && !bc.live() && !bp.live()) {
      // the cur block is outside the range too: a later step multiplies its P by V
      p_cur[0] = f16x8{};
      p_cur[1] = f16x8{};
      return;
    }
    if (!bc.live() || bc.masked()) mask_scores(s_cur, bc);
    if (bn.kind() == BIAS_TWO)
      s_init(s_next, bn, tst, nblk, KTwo{});
    else if (bn.kind() == BIAS_GENERAL)
      s_init(s_next, bn, tst, nblk, KGen{});
    else
      s_init(s_next, bn, tst, nblk, KConst{});
    fused(s_next, kst, nblk, s_cur, p_cur, p_prev, vst, pblk);
  };

  // Tile t's blocks are 2t (blk 0) and 2t + 1 (blk 1).  Iteration t runs steps 2t + 1 and
  // 2t + 2, which read only K tile t + 1 and V tile t; the loads issued in iteration t
  // (K of t + 2, V of t + 1) go to the stages that iteration t - 1 finished reading, and
  // the barrier that opens iteration t + 1 waits for them.
  f32x16 sc0 = {}, sc1 = {};        // scores of the even / odd block in flight
  f16x8 pe[2] = {}, po[2] = {};     // P^T of the even / odd block
  BlockInfo cur0{}, cur1{}, nxt0{}, nxt1{};
  auto iteration = [&](int t, auto r_c) __attribute__((always_inline)) {  // r_c = t mod NS
    constexpr int R = decltype(r_c)::value;
    constexpr int KR = (R + 1) % NS;
    // wait for this wave's loads of batch t - LEAD and its LDS reads, then for every wave
    __builtin_amdgcn_s_waitcnt(((LEAD - 1) * LPW) | (7 << 4));  // vmcnt(N) expcnt(7) lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // next 64 blocks of the table, once every 32 tiles (before the batch, so that the
    // wait for the timestamp ranges is not a wait for the batch)
    if (2 * (t + 1) >= cbase + 64) build_table(cbase + 64);
    batch(t, r_c, std::integral_constant<int, 0>{});
    cur0 = nxt0;
    cur1 = nxt1;
    const unsigned char *kst = kbuf(std::integral_constant<int, KR>{});  // K, ts of tile t + 1
    const int32_t *tst = tbuf(std::integral_constant<int, KR>{});
    nxt0 = fetch(2 * t + 2);
    nxt1 = fetch(2 * t + 3);
    const unsigned char *vst = vbuf(r_c);                                 // V of tile t
    step(sc0, nxt0, kst, tst, 0, sc1, po, cur1, pe, cur0, vst, 0);
    batch(t, r_c, std::integral_constant<int, 1>{});
    step(sc1, nxt1, kst, tst, 1, sc0, pe, nxt0, po, cur1, vst, 1);
  };
  for (int t = -1; t < n_tiles; t += NS) {
    iteration(t, CLast{});
    if (t + 1 < n_tiles) iteration(t + 1, C0{});
    if constexpr (NS == 3)
      if (t + 2 < n_tiles) iteration(t + 2, C1{});
  }
  __builtin_amdgcn_s_waitcnt(7 << 4);  // drain the dummy batches before the stores

  // epilogue: lane holds query lrow, features 32f + 8g + 4*half + 0..3 (the other half of
  // the head's features sits in lane ^ 32)
#pragma unroll
  for (int f = 0; f < FT; ++f) acc_o[f] *= kNegLn2;
  if (p.cn == nullptr) {  // the raw aggregation, fp32 rows
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
  } else {
    // Inside the layer the aggregation only feeds the LayerNorm of equation 3, taken over
    // all H dv features of a row.  This head's part is summarised by its mean and biased
    // variance (two passes over registers) and stored standardised with them, as fp16
    // (|value| <= sqrt(DH)); f2 combines the heads' statistics exactly and rebuilds the
    // normalised row from these parts.
    float sum = 0.f;
#pragma unroll
    for (int f = 0; f < FT; ++f)
#pragma unroll
      for (int i = 0; i < 16; ++i) sum += acc_o[f][i];
    sum += __shfl_xor(sum, 32, 64);
    const float mean = sum * (1.0f / DH);
    float m2 = 0.f;
#pragma unroll
    for (int f = 0; f < FT; ++f)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float d = acc_o[f][i] - mean;
        m2 += d * d;
      }
    m2 += __shfl_xor(m2, 32, 64);
    const float var = m2 * (1.0f / DH);
    const float inv = var > 0.f ? __builtin_amdgcn_rsqf(var) : 0.f;
    if (q_ok) {
      uint16_t *crow = p.cn + (int64_t)(s0 + qi) * p.out_stride + h * DH + half * 4;
#pragma unroll
      for (int f = 0; f < FT; ++f)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const u32x2 v = {pack_f16((acc_o[f][4 * g] - mean) * inv, (acc_o[f][4 * g + 1] - mean) * inv),
                           pack_f16((acc_o[f][4 * g + 2] - mean) * inv, (acc_o[f][4 * g + 3] - mean) * inv)};
          *reinterpret_cast<u32x2 *>(crow + f * 32 + g * 8) = v;
        }
      if (half == 0) p.stats[(int64_t)(s0 + qi) * p.num_heads + h] = float2{mean, var};
    }
  }
  if (p.clk != nullptr && blockIdx.x < kClockSlots && threadIdx.x == 0) {
    const uint64_t clk1 = __builtin_amdgcn_s_memtime(), rt1 = __builtin_amdgcn_s_memrealtime();
    // added up over launches (one writer per slot and launch, launches in stream order)
    p.clk[2 * blockIdx.x] += clk1 - clk0;
    p.clk[2 * blockIdx.x + 1] += rt1 - rt0;
  }
}

template <int DH, int MASK, int NW, bool PRE>
hipError_t launch_one(const AttnArgs &a, int64_t cap, hipStream_t stream) {
  const dim3 grid((unsigned)(cap * a.num_heads), 1u);
  attn_kernel<DH, MASK, NW, PRE><<<grid, dim3(64 * NW), 0, stream>>>(a);
  return hipGetLastError();
}

template <int DH, int NW>
hipError_t launch_dh(const AttnArgs &a, int64_t cap, hipStream_t stream) {
  if (a.mask != 0) return launch_one<DH, 1, NW, true>(a, cap, stream);
  return a.p_offsets != nullptr ? launch_one<DH, 0, NW, true>(a, cap, stream)
                                : launch_one<DH, 0, NW, false>(a, cap, stream);
}

}  // namespace

hipError_t launch_attention(const AttnArgs &a, int dh, int max_seq_len, int64_t cap,
                            hipStream_t stream) {
  if (cap <= 0 || a.num_heads <= 0) return hipSuccess;
  static_assert(kAttnBlockMMin == 128, "4-wave workgroups");
  (void)max_seq_len;
  switch (dh) {
    case 32: return launch_dh<32, 4>(a, cap, stream);
    case 64: return launch_dh<64, 4>(a, cap, stream);
    case 128: return launch_dh<128, 4>(a, cap, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace hstu
