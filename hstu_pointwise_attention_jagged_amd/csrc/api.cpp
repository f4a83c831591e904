// C ABI of libhstu: argument checks, workspace layout, launch order and optional
// per-kernel event timing.  Every numeric step runs in the HIP kernels; this file only
// validates, carves the caller's workspace and enqueues launches on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <utility>
#include <vector>

#include "../../include/hstu.h"
#include "kernels.h"

using namespace hstu;

namespace {

thread_local int g_last_hip_error = 0;

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// ---------------------------------------------------------------- profiling ---------
uint64_t *clock_samples();  // below: this device's copy of the clock-sample array
constexpr int kNumKernels = 5;
const char *kKernelNames[kNumKernels] = {"schedule", "f1_gemm_silu", "attention", "f2_prep",
                                         "f2_gemm"};

struct ProfRecord {
  int id;
  hipEvent_t start, stop;
};

std::mutex g_prof_mu;
int g_prof_mask = 0;  // bit k: time the launches of kernel id k
std::vector<ProfRecord> g_prof_records;
std::vector<hipEvent_t> g_event_pool;

hipEvent_t pool_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Runs `launch` on `stream`, bracketed by events when profiling is on.
template <typename F>
hipError_t timed(int id, hipStream_t stream, F &&launch) {
  hipEvent_t a = nullptr, b = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if ((g_prof_mask >> id) & 1) {
      a = pool_event();
      b = pool_event();
    }
  }
  if (a && b) (void)hipEventRecord(a, stream);
  hipError_t err = launch();
  if (a && b) {
    (void)hipEventRecord(b, stream);
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_records.push_back({id, a, b});
  }
  return err;
}

bool attention_profiled() {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  return (g_prof_mask >> 2) & 1;
}

hstu_status_t hip_fail(hipError_t e) {
  g_last_hip_error = (int)e;
  return HSTU_ERR_HIP;
}

// ---------------------------------------------------------------- checks ------------
// Shape rules of the attention kernel alone.
hstu_status_t check_attn_dims(const hstu_dims_t *d) {
  if (d == nullptr) return HSTU_ERR_INVALID_ARG;
  if (d->num_heads <= 0 || d->dqk <= 0 || d->dv <= 0) return HSTU_ERR_INVALID_ARG;
  if (d->pos_buckets < 1 || d->time_buckets < 1) return HSTU_ERR_INVALID_ARG;
  if (d->rab_heads != 1 && d->rab_heads != d->num_heads) return HSTU_ERR_INVALID_ARG;
  if (d->dqk != d->dv) return HSTU_ERR_UNSUPPORTED;
  if (d->dqk != 32 && d->dqk != 64 && d->dqk != 128) return HSTU_ERR_UNSUPPORTED;
  if (d->pos_buckets > 1024 || d->time_buckets > 64) return HSTU_ERR_UNSUPPORTED;
  return HSTU_OK;
}

// Shape rules of the whole layer (projections and norm-gate too).
hstu_status_t check_dims(const hstu_dims_t *d) {
  if (d == nullptr) return HSTU_ERR_INVALID_ARG;
  if (d->d_model <= 0 || d->num_heads <= 0 || d->dqk <= 0 || d->dv <= 0) return HSTU_ERR_INVALID_ARG;
  if (d->pos_buckets < 1 || d->time_buckets < 1) return HSTU_ERR_INVALID_ARG;
  if (d->rab_heads != 1 && d->rab_heads != d->num_heads) return HSTU_ERR_INVALID_ARG;
  if (!(d->ln_eps >= 0.0f) || !std::isfinite(d->ln_eps)) return HSTU_ERR_INVALID_ARG;
  if (d->dqk != d->dv) return HSTU_ERR_UNSUPPORTED;
  if (d->dqk != 32 && d->dqk != 64 && d->dqk != 128) return HSTU_ERR_UNSUPPORTED;
  if (d->d_model % 64 != 0 || d->d_model > kGemmMaxK) return HSTU_ERR_UNSUPPORTED;
  const int64_t hdv = (int64_t)d->num_heads * d->dv;
  if (hdv % 64 != 0 || hdv > 2048) return HSTU_ERR_UNSUPPORTED;
  if (d->pos_buckets > 1024 || d->time_buckets > 64) return HSTU_ERR_UNSUPPORTED;
  return HSTU_OK;
}

hstu_status_t check_seq(const hstu_jagged_t *s) {
  if (s == nullptr) return HSTU_ERR_INVALID_ARG;
  if (s->batch < 0 || s->total_tokens < 0 || s->max_seq_len < 0) return HSTU_ERR_INVALID_ARG;
  if (s->seq_offsets == nullptr) return HSTU_ERR_INVALID_ARG;
  if (s->batch == 0 && s->total_tokens != 0) return HSTU_ERR_INVALID_ARG;
  if (s->total_tokens > 0 && s->max_seq_len == 0) return HSTU_ERR_INVALID_ARG;
  return HSTU_OK;
}

// The attention kernel addresses one sequence's key rows through 32-bit buffer offsets:
// (longest sequence + one stage) rows of `row_elems` fp16 values must stay below 2^31 bytes.
bool rows_addressable(int max_seq_len, int64_t row_elems) {
  return ((int64_t)max_seq_len + 64) * row_elems * 2 < ((int64_t)1 << 31);
}

// Attention scratch: work count, work list, per-token key-block timestamp ranges of the
// batch and of its prefix (if any).
size_t attn_ws_bytes(const hstu_jagged_t *s, const hstu_jagged_t *pre) {
  const int64_t cap = attn_work_capacity(s->batch, s->total_tokens);
  size_t bytes = kAlign + align_up((size_t)cap * 2 * sizeof(int32_t));
  bytes += align_up((size_t)s->total_tokens * 8);
  if (pre != nullptr) bytes += align_up((size_t)pre->total_tokens * 8);
  return bytes;
}

// Layer scratch: the attention's standardised per-head output (fp16 [T][H dv]) and its
// per-(row, head) statistics (float2 [T][H]), w2 as fp16 and gamma | beta as fp16 for f2,
// then the attention scratch.
size_t layer_ws_bytes(const hstu_dims_t *d, const hstu_jagged_t *s, const hstu_jagged_t *pre) {
  const size_t T = (size_t)s->total_tokens, hdv = (size_t)d->num_heads * d->dv;
  return align_up(T * hdv * sizeof(uint16_t)) + align_up(T * d->num_heads * 8) +
         align_up((size_t)d->d_model * hdv * sizeof(uint16_t)) + align_up(2 * hdv * sizeof(uint16_t)) +
         attn_ws_bytes(s, pre);
}

// A stack adds one [T][d] bf16 activation buffer (the layers alternate between it and y).
size_t stack_ws_bytes(const hstu_dims_t *d, const hstu_jagged_t *s, const hstu_jagged_t *pre) {
  return layer_ws_bytes(d, s, pre) + align_up((size_t)s->total_tokens * d->d_model * sizeof(uint16_t));
}

struct LayerWs {
  float *o;         // raw attention output (attention alone, layer backward)
  uint16_t *cn;     // or: standardised per-head output and its statistics (layer forward)
  float2 *stats;
  uint16_t *w2h;    // w2 as fp16
  uint16_t *gb;     // gamma | beta as fp16
  int32_t *work;
  int32_t *n_work;
  int2 *kstat;
  int2 *p_kstat;
};

void carve_attn(char *p, const hstu_jagged_t *s, const hstu_jagged_t *pre, LayerWs &w) {
  const int64_t cap = attn_work_capacity(s->batch, s->total_tokens);
  w.n_work = (int32_t *)p;
  p += kAlign;
  w.work = (int32_t *)p;
  p += align_up((size_t)cap * 2 * sizeof(int32_t));
  w.kstat = (int2 *)p;
  p += align_up((size_t)s->total_tokens * 8);
  w.p_kstat = pre != nullptr ? (int2 *)p : nullptr;
}

LayerWs carve_layer(void *ws, const hstu_dims_t *d, const hstu_jagged_t *s,
                    const hstu_jagged_t *pre) {
  const size_t T = (size_t)s->total_tokens, hdv = (size_t)d->num_heads * d->dv;
  char *p = (char *)ws;
  LayerWs w{};
  w.cn = (uint16_t *)p;
  p += align_up(T * hdv * sizeof(uint16_t));
  w.stats = (float2 *)p;
  p += align_up(T * d->num_heads * 8);
  w.w2h = (uint16_t *)p;
  p += align_up((size_t)d->d_model * hdv * sizeof(uint16_t));
  w.gb = (uint16_t *)p;
  p += align_up(2 * hdv * sizeof(uint16_t));
  carve_attn(p, s, pre, w);
  return w;
}

// Key-block timestamp ranges for the batch and its prefix, when the time term is on.
hipError_t launch_stats(const AttnArgs &aa, const hstu_jagged_t *s, const hstu_jagged_t *pre,
                        hipStream_t st, bool force = false) {
  if ((!force && aa.rab_time == nullptr) || s->timestamps == nullptr) return hipSuccess;
  hipError_t e = launch_block_stats(s->timestamps, s->seq_offsets, s->batch, s->max_seq_len,
                                    const_cast<int2 *>(aa.kstat), st);
  if (e == hipSuccess && pre != nullptr && pre->timestamps != nullptr && pre->total_tokens > 0)
    e = launch_block_stats(pre->timestamps, pre->seq_offsets, pre->batch, pre->max_seq_len,
                           const_cast<int2 *>(aa.p_kstat), st);
  return e;
}

hstu_status_t check_ws(void *ws, size_t have, size_t need) {
  if (need > 0 && (ws == nullptr || have < need)) return HSTU_ERR_WORKSPACE;
  if (((uintptr_t)ws & (kAlign - 1)) != 0) return HSTU_ERR_WORKSPACE;
  return HSTU_OK;
}

AttnArgs attn_args(const hstu_dims_t *d, const float *rab_pos, const float *rab_time,
                   const hstu_jagged_t *s, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                   int64_t stride, float *out, const LayerWs &w) {
  AttnArgs a{};
  a.offsets = s->seq_offsets;
  a.ts = s->timestamps;
  a.q = q;
  a.k = k;
  a.v = v;
  a.stride = stride;
  a.rab_pos = rab_pos;
  a.rab_time = rab_time;
  a.pos_buckets = d->pos_buckets;
  a.time_buckets = d->time_buckets;
  a.rab_per_head = d->rab_heads == d->num_heads && d->num_heads > 1;
  a.out = out;
  a.out_stride = (int64_t)d->num_heads * d->dv;
  a.cn = w.cn;
  a.stats = w.stats;
  a.work = w.work;
  a.n_work = w.n_work;
  a.kstat = w.kstat;
  a.p_kstat = w.p_kstat;
  a.num_heads = d->num_heads;
  a.mask = 0;
  return a;
}

// Jagged tile schedule and key-block timestamp ranges of a batch (and its prefix).  They
// depend only on the batch, so a stack of layers builds them once; `all_stats` asks for
// the ranges whenever timestamps exist (a later layer of a stack may use the time term).
hstu_status_t run_setup(const hstu_jagged_t *s, const AttnArgs &aa, const LayerWs &lw,
                        const hstu_jagged_t *pre, bool all_stats, hipStream_t st) {
  const int max_prefix = pre != nullptr ? pre->max_seq_len : 0;
  hipError_t e = timed(0, st, [&] {
    return launch_schedule(s->seq_offsets, aa.p_offsets, s->batch, aa.mask, s->max_seq_len,
                           max_prefix, lw.work, lw.n_work, st);
  });
  if (e != hipSuccess) return hip_fail(e);
  e = timed(0, st, [&] { return launch_stats(aa, s, pre, st, all_stats); });
  if (e != hipSuccess) return hip_fail(e);
  return HSTU_OK;
}

// f1 -> attention -> f2 (LayerNorm and gate in its staging) for one batch whose attention
// args are ready.
hstu_status_t run_layer(const hstu_dims_t *d, const hstu_weights_t *w, const hstu_jagged_t *s,
                        const uint16_t *x, uint16_t *y, uint16_t *uvqk, const AttnArgs &aa,
                        const LayerWs &lw, const hstu_jagged_t *pre, hipStream_t st,
                        bool setup = true) {
  const int T = s->total_tokens;
  const int hdv = d->num_heads * d->dv;
  const int n1 = 2 * d->num_heads * (d->dqk + d->dv);
  hipError_t e;
  if (setup) {
    const hstu_status_t r = run_setup(s, aa, lw, pre, false, st);
    if (r != HSTU_OK) return r;
  }
  const bool affine = w->ln_gamma != nullptr || w->ln_beta != nullptr;
  // T may be a capacity: the GEMMs read the true row count, seq_offsets[B], on the device
  const int32_t *t_dev = s->seq_offsets + s->batch;
  // f1, with the f2 operand conversion (w2, gamma, beta to fp16) riding along
  W2Prep prep;
  prep.w2 = w->w2;
  prep.n_w = (int64_t)d->d_model * hdv;
  prep.gamma = w->ln_gamma;
  prep.beta = w->ln_beta;
  prep.K = hdv;
  prep.w2h = lw.w2h;
  prep.gb = affine ? reinterpret_cast<_Float16 *>(lw.gb) : nullptr;
  e = timed(1, st, [&] {
    return launch_gemm(x, w->w1, w->b1, uvqk, T, n1, d->d_model, ACT_SILU, OUT_F16, st, t_dev, &prep);
  });
  if (e != hipSuccess) return hip_fail(e);
  const int64_t cap = attn_work_capacity(s->batch, T);
  AttnArgs at = aa;
  if (attention_profiled()) at.clk = clock_samples();  // lifetime clocks of the first workgroups
  e = timed(2, st, [&] { return launch_attention(at, d->dqk, s->max_seq_len, cap, st); });
  if (e != hipSuccess) return hip_fail(e);
  GateGemmArgs ga{};
  ga.w = lw.w2h;
  ga.c = lw.cn;
  ga.u = uvqk;  // U is the first H dv columns of each row
  ga.u_stride = n1;
  ga.stats = lw.stats;
  ga.gb = affine ? reinterpret_cast<const _Float16 *>(lw.gb) : nullptr;
  ga.bias = w->b2;
  ga.out = y;
  ga.m_dev = t_dev;
  ga.M = T;
  ga.N = d->d_model;
  ga.K = hdv;
  ga.H = d->num_heads;
  ga.dv = d->dv;
  ga.eps = d->ln_eps;
  e = timed(4, st, [&] { return launch_gate_gemm(ga, affine, st); });
  if (e != hipSuccess) return hip_fail(e);
  return HSTU_OK;
}

hstu_status_t check_weights(const hstu_weights_t *w) {
  if (w == nullptr || w->w1 == nullptr || w->w2 == nullptr) return HSTU_ERR_INVALID_ARG;
  if (!aligned16(w->w1) || !aligned16(w->w2)) return HSTU_ERR_INVALID_ARG;
  if ((w->b1 && !aligned16(w->b1)) || (w->b2 && !aligned16(w->b2))) return HSTU_ERR_INVALID_ARG;
  return HSTU_OK;
}

}  // namespace

extern "C" {

size_t hstu_layer_workspace_bytes(const hstu_dims_t *dims, const hstu_jagged_t *seq) {
  if (check_dims(dims) != HSTU_OK || check_seq(seq) != HSTU_OK) return 0;
  return layer_ws_bytes(dims, seq, nullptr);
}

size_t hstu_mfalcon_workspace_bytes(const hstu_dims_t *dims, const hstu_jagged_t *hist,
                                    const hstu_jagged_t *cand) {
  if (check_dims(dims) != HSTU_OK || check_seq(hist) != HSTU_OK || check_seq(cand) != HSTU_OK)
    return 0;
  return layer_ws_bytes(dims, cand, hist);
}

size_t hstu_attn_workspace_bytes(const hstu_dims_t *dims, const hstu_jagged_t *seq,
                                 const hstu_jagged_t *prefix_seq) {
  if (check_attn_dims(dims) != HSTU_OK || check_seq(seq) != HSTU_OK) return 0;
  if (prefix_seq != nullptr && check_seq(prefix_seq) != HSTU_OK) return 0;
  return attn_ws_bytes(seq, prefix_seq);
}

hstu_status_t hstu_layer_fwd(const hstu_dims_t *dims, const hstu_weights_t *w,
                             const hstu_jagged_t *seq, const uint16_t *x, uint16_t *y,
                             uint16_t *uvqk, void *ws, size_t ws_bytes, void *stream) {
  hstu_status_t st;
  if ((st = check_dims(dims)) != HSTU_OK) return st;
  if ((st = check_seq(seq)) != HSTU_OK) return st;
  if ((st = check_weights(w)) != HSTU_OK) return st;
  if (seq->total_tokens > 0 && (x == nullptr || y == nullptr || uvqk == nullptr))
    return HSTU_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(y) || !aligned16(uvqk)) return HSTU_ERR_INVALID_ARG;
  if ((void *)x == (void *)y) return HSTU_ERR_INVALID_ARG;
  if (seq->batch == 0 || seq->total_tokens == 0) return HSTU_OK;
  if ((st = check_ws(ws, ws_bytes, layer_ws_bytes(dims, seq, nullptr))) != HSTU_OK) return st;
  if (!rows_addressable(seq->max_seq_len, 2 * (int64_t)dims->num_heads * (dims->dqk + dims->dv)))
    return HSTU_ERR_UNSUPPORTED;

  const LayerWs lw = carve_layer(ws, dims, seq, nullptr);
  const int hdv = dims->num_heads * dims->dv, hqk = dims->num_heads * dims->dqk;
  const int64_t n1 = 2 * (int64_t)(hdv + hqk);
  AttnArgs aa = attn_args(dims, w->rab_pos, w->rab_time, seq, uvqk + 2 * hdv,
                          uvqk + 2 * hdv + hqk, uvqk + hdv, n1, lw.o, lw);
  return run_layer(dims, w, seq, x, y, uvqk, aa, lw, nullptr, (hipStream_t)stream);
}

hstu_status_t hstu_layer_fwd_train(const hstu_dims_t *dims, const hstu_weights_t *w,
                                   const hstu_jagged_t *seq, const uint16_t *x, uint16_t *y,
                                   uint16_t *uvqk, uint16_t *cn, float *stats, void *ws,
                                   size_t ws_bytes, void *stream) {
  hstu_status_t st;
  if ((st = check_dims(dims)) != HSTU_OK) return st;
  if ((st = check_seq(seq)) != HSTU_OK) return st;
  if ((st = check_weights(w)) != HSTU_OK) return st;
  if (seq->total_tokens > 0 &&
      (x == nullptr || y == nullptr || uvqk == nullptr || cn == nullptr || stats == nullptr))
    return HSTU_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(y) || !aligned16(uvqk) || !aligned16(cn) || !aligned16(stats))
    return HSTU_ERR_INVALID_ARG;
  if ((void *)x == (void *)y || (void *)cn == (void *)y || (void *)cn == (void *)uvqk ||
      (void *)stats == (void *)y || (void *)stats == (void *)uvqk || (void *)stats == (void *)cn)
    return HSTU_ERR_INVALID_ARG;
  if (seq->batch == 0 || seq->total_tokens == 0) return HSTU_OK;
  if ((st = check_ws(ws, ws_bytes, layer_ws_bytes(dims, seq, nullptr))) != HSTU_OK) return st;
  if (!rows_addressable(seq->max_seq_len, 2 * (int64_t)dims->num_heads * (dims->dqk + dims->dv)))
    return HSTU_ERR_UNSUPPORTED;

  LayerWs lw = carve_layer(ws, dims, seq, nullptr);
  lw.cn = cn;  // the attention's standardised output and statistics go to the caller
  lw.stats = reinterpret_cast<float2 *>(stats);
  const int hdv = dims->num_heads * dims->dv, hqk = dims->num_heads * dims->dqk;
  const int64_t n1 = 2 * (int64_t)(hdv + hqk);
  AttnArgs aa = attn_args(dims, w->rab_pos, w->rab_time, seq, uvqk + 2 * hdv,
                          uvqk + 2 * hdv + hqk, uvqk + hdv, n1, lw.o, lw);
  return run_layer(dims, w, seq, x, y, uvqk, aa, lw, nullptr, (hipStream_t)stream);
}

hstu_status_t hstu_layer_fwd_mfalcon(const hstu_dims_t *dims, const hstu_weights_t *w,
                                     const hstu_jagged_t *hist, const uint16_t *hist_uvqk,
                                     const hstu_jagged_t *cand, const uint16_t *x_cand,
                                     uint16_t *y_cand, uint16_t *uvqk_cand, void *ws,
                                     size_t ws_bytes, void *stream) {
  hstu_status_t st;
  if ((st = check_dims(dims)) != HSTU_OK) return st;
  if ((st = check_seq(hist)) != HSTU_OK) return st;
  if ((st = check_seq(cand)) != HSTU_OK) return st;
  if ((st = check_weights(w)) != HSTU_OK) return st;
  if (hist->batch != cand->batch) return HSTU_ERR_INVALID_ARG;
  if (hist->total_tokens > 0 && hist_uvqk == nullptr) return HSTU_ERR_INVALID_ARG;
  if (cand->total_tokens > 0 && (x_cand == nullptr || y_cand == nullptr || uvqk_cand == nullptr))
    return HSTU_ERR_INVALID_ARG;
  if (!aligned16(hist_uvqk) || !aligned16(x_cand) || !aligned16(y_cand) || !aligned16(uvqk_cand))
    return HSTU_ERR_INVALID_ARG;
  if ((void *)x_cand == (void *)y_cand) return HSTU_ERR_INVALID_ARG;
  if ((cand->timestamps == nullptr) != (hist->timestamps == nullptr)) return HSTU_ERR_INVALID_ARG;
  if (cand->batch == 0 || cand->total_tokens == 0) return HSTU_OK;
  if ((st = check_ws(ws, ws_bytes, layer_ws_bytes(dims, cand, hist))) != HSTU_OK) return st;
  {
    const int64_t n1 = 2 * (int64_t)dims->num_heads * (dims->dqk + dims->dv);
    if (!rows_addressable(cand->max_seq_len, n1) || !rows_addressable(hist->max_seq_len, n1))
      return HSTU_ERR_UNSUPPORTED;
  }

  const LayerWs lw = carve_layer(ws, dims, cand, hist);
  const int hdv = dims->num_heads * dims->dv, hqk = dims->num_heads * dims->dqk;
  const int64_t n1 = 2 * (int64_t)(hdv + hqk);
  AttnArgs aa = attn_args(dims, w->rab_pos, w->rab_time, cand, uvqk_cand + 2 * hdv,
                          uvqk_cand + 2 * hdv + hqk, uvqk_cand + hdv, n1, lw.o, lw);
  aa.mask = 1;
  aa.p_offsets = hist->seq_offsets;
  aa.p_ts = hist->timestamps;
  aa.pk = hist_uvqk + 2 * hdv + hqk;
  aa.pv = hist_uvqk + hdv;
  aa.p_stride = n1;
  return run_layer(dims, w, cand, x_cand, y_cand, uvqk_cand, aa, lw, hist, (hipStream_t)stream);
}

size_t hstu_stack_workspace_bytes(const hstu_dims_t *dims, const hstu_jagged_t *seq) {
  if (check_dims(dims) != HSTU_OK || check_seq(seq) != HSTU_OK) return 0;
  return stack_ws_bytes(dims, seq, nullptr);
}

size_t hstu_stack_mfalcon_workspace_bytes(const hstu_dims_t *dims, const hstu_jagged_t *hist,
                                          const hstu_jagged_t *cand) {
  if (check_dims(dims) != HSTU_OK || check_seq(hist) != HSTU_OK || check_seq(cand) != HSTU_OK)
    return 0;
  return stack_ws_bytes(dims, cand, hist);
}

hstu_status_t hstu_stack_fwd(const hstu_dims_t *dims, int32_t n_layers, const hstu_weights_t *w,
                             const hstu_jagged_t *seq, const uint16_t *x, uint16_t *y,
                             uint16_t *uvqk, int32_t keep_caches, void *ws, size_t ws_bytes,
                             void *stream) {
  hstu_status_t st;
  if ((st = check_dims(dims)) != HSTU_OK) return st;
  if ((st = check_seq(seq)) != HSTU_OK) return st;
  if (n_layers < 1 || w == nullptr) return HSTU_ERR_INVALID_ARG;
  for (int l = 0; l < n_layers; ++l)
    if ((st = check_weights(&w[l])) != HSTU_OK) return st;
  if (seq->total_tokens > 0 && (x == nullptr || y == nullptr || uvqk == nullptr))
    return HSTU_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(y) || !aligned16(uvqk)) return HSTU_ERR_INVALID_ARG;
  if ((void *)x == (void *)y) return HSTU_ERR_INVALID_ARG;
  if (seq->batch == 0 || seq->total_tokens == 0) return HSTU_OK;
  if ((st = check_ws(ws, ws_bytes, stack_ws_bytes(dims, seq, nullptr))) != HSTU_OK) return st;
  const int hdv = dims->num_heads * dims->dv, hqk = dims->num_heads * dims->dqk;
  const int64_t n1 = 2 * (int64_t)(hdv + hqk);
  if (!rows_addressable(seq->max_seq_len, n1)) return HSTU_ERR_UNSUPPORTED;

  hipStream_t sst = (hipStream_t)stream;
  const LayerWs lw = carve_layer(ws, dims, seq, nullptr);
  uint16_t *act = (uint16_t *)((char *)ws + layer_ws_bytes(dims, seq, nullptr));
  const size_t cache = (size_t)seq->total_tokens * n1;
  auto args = [&](int l) {
    uint16_t *u = uvqk + (keep_caches ? (size_t)l * cache : 0);
    return attn_args(dims, w[l].rab_pos, w[l].rab_time, seq, u + 2 * hdv, u + 2 * hdv + hqk,
                     u + hdv, n1, lw.o, lw);
  };
  if ((st = run_setup(seq, args(0), lw, nullptr, true, sst)) != HSTU_OK) return st;
  const uint16_t *in = x;
  for (int l = 0; l < n_layers; ++l) {
    // the last layer writes y; earlier layers alternate so that no layer reads its output
    uint16_t *out = ((n_layers - 1 - l) % 2 == 0) ? y : act;
    uint16_t *u = uvqk + (keep_caches ? (size_t)l * cache : 0);
    if ((st = run_layer(dims, &w[l], seq, in, out, u, args(l), lw, nullptr, sst, false)) != HSTU_OK)
      return st;
    in = out;
  }
  return HSTU_OK;
}

hstu_status_t hstu_stack_fwd_mfalcon(const hstu_dims_t *dims, int32_t n_layers,
                                     const hstu_weights_t *w, const hstu_jagged_t *hist,
                                     const uint16_t *hist_uvqk, const hstu_jagged_t *cand,
                                     const uint16_t *x_cand, uint16_t *y_cand, uint16_t *uvqk_cand,
                                     void *ws, size_t ws_bytes, void *stream) {
  hstu_status_t st;
  if ((st = check_dims(dims)) != HSTU_OK) return st;
  if ((st = check_seq(hist)) != HSTU_OK) return st;
  if ((st = check_seq(cand)) != HSTU_OK) return st;
  if (n_layers < 1 || w == nullptr) return HSTU_ERR_INVALID_ARG;
  for (int l = 0; l < n_layers; ++l)
    if ((st = check_weights(&w[l])) != HSTU_OK) return st;
  if (hist->batch != cand->batch) return HSTU_ERR_INVALID_ARG;
  if (hist->total_tokens > 0 && hist_uvqk == nullptr) return HSTU_ERR_INVALID_ARG;
  if (cand->total_tokens > 0 && (x_cand == nullptr || y_cand == nullptr || uvqk_cand == nullptr))
    return HSTU_ERR_INVALID_ARG;
  if (!aligned16(hist_uvqk) || !aligned16(x_cand) || !aligned16(y_cand) || !aligned16(uvqk_cand))
    return HSTU_ERR_INVALID_ARG;
  if ((void *)x_cand == (void *)y_cand) return HSTU_ERR_INVALID_ARG;
  if ((cand->timestamps == nullptr) != (hist->timestamps == nullptr)) return HSTU_ERR_INVALID_ARG;
  if (cand->batch == 0 || cand->total_tokens == 0) return HSTU_OK;
  if ((st = check_ws(ws, ws_bytes, stack_ws_bytes(dims, cand, hist))) != HSTU_OK) return st;
  const int hdv = dims->num_heads * dims->dv, hqk = dims->num_heads * dims->dqk;
  const int64_t n1 = 2 * (int64_t)(hdv + hqk);
  if (!rows_addressable(cand->max_seq_len, n1) || !rows_addressable(hist->max_seq_len, n1))
    return HSTU_ERR_UNSUPPORTED;

  hipStream_t sst = (hipStream_t)stream;
  const LayerWs lw = carve_layer(ws, dims, cand, hist);
  uint16_t *act = (uint16_t *)((char *)ws + layer_ws_bytes(dims, cand, hist));
  const size_t cache = (size_t)hist->total_tokens * n1;
  auto args = [&](int l) {
    AttnArgs aa = attn_args(dims, w[l].rab_pos, w[l].rab_time, cand, uvqk_cand + 2 * hdv,
                            uvqk_cand + 2 * hdv + hqk, uvqk_cand + hdv, n1, lw.o, lw);
    const uint16_t *hu = hist_uvqk + (size_t)l * cache;
    aa.mask = 1;
    aa.p_offsets = hist->seq_offsets;
    aa.p_ts = hist->timestamps;
    aa.pk = hu + 2 * hdv + hqk;
    aa.pv = hu + hdv;
    aa.p_stride = n1;
    return aa;
  };
  if ((st = run_setup(cand, args(0), lw, hist, true, sst)) != HSTU_OK) return st;
  const uint16_t *in = x_cand;
  for (int l = 0; l < n_layers; ++l) {
    uint16_t *out = ((n_layers - 1 - l) % 2 == 0) ? y_cand : act;
    if ((st = run_layer(dims, &w[l], cand, in, out, uvqk_cand, args(l), lw, hist, sst, false)) !=
        HSTU_OK)
      return st;
    in = out;
  }
  return HSTU_OK;
}

// The schedule and block statistics of the forward, then the fp16 copy of d_out and the
// word that holds max |d_out|.
// Per-work-item bins of the bias-table gradients: [H][cap][pos_buckets + time_buckets].
static size_t rab_part_bytes(const hstu_dims_t *d, const hstu_jagged_t *s) {
  return align_up((size_t)attn_work_capacity(s->batch, s->total_tokens) * d->num_heads *
                  (d->pos_buckets + d->time_buckets) * sizeof(float));
}

static size_t attn_bwd_ws_bytes(const hstu_dims_t *d, const hstu_jagged_t *s) {
  return attn_ws_bytes(s, nullptr) +
         align_up((size_t)s->total_tokens * d->num_heads * d->dv * sizeof(uint16_t)) + kAlign +
         rab_part_bytes(d, s);
}

// Stored dS of the attention backward: per head, an upper bound on the 32 x 32 blocks of
// every sequence's causal triangle that the host can form from T, B and the longest
// length L: the sum of nb (nb + 1) / 2 with nb = ceil(n / 32) <= ceil(L / 32) and the sum
// of nb at most ceil(T / 32) + B.  0 when the buffer would pass kDsCapBytes (then the dQ
// kernel forms dS again).
constexpr size_t kDsCapBytes = (size_t)32 << 30;

static int64_t ds_head_blocks(const hstu_jagged_t *s) {
  const int64_t nb_max = ((int64_t)s->max_seq_len + 31) / 32;
  return (((int64_t)s->total_tokens + 31) / 32 + s->batch) * (nb_max + 1) / 2 + 1;
}

static size_t ds_bytes(const hstu_dims_t *d, const hstu_jagged_t *s) {
  if (s->total_tokens == 0) return 0;
  const size_t bytes = align_up((size_t)(s->batch + 1) * sizeof(int64_t)) + 2048 +
                       align_up((size_t)ds_head_blocks(s) * d->num_heads * 2048);
  return bytes <= kDsCapBytes ? bytes : 0;
}

size_t hstu_attn_bwd_workspace_bytes(const hstu_dims_t *dims, const hstu_jagged_t *seq) {
  if (check_attn_dims(dims) != HSTU_OK || check_seq(seq) != HSTU_OK) return 0;
  return attn_bwd_ws_bytes(dims, seq) + ds_bytes(dims, seq);
}

size_t hstu_attn_bwd_min_workspace_bytes(const hstu_dims_t *dims, const hstu_jagged_t *seq) {
  if (check_attn_dims(dims) != HSTU_OK || check_seq(seq) != HSTU_OK) return 0;
  return attn_bwd_ws_bytes(dims, seq);
}

// Points a at the stored-dS region that follows `base` when the workspace holds it.
static void attach_ds(AttnBwdArgs &a, const hstu_dims_t *d, const hstu_jagged_t *s, char *base,
                      size_t have) {
  const size_t need = ds_bytes(d, s);
  if (need == 0 || have < need) return;
  a.tri_base = (int64_t *)base;
  a.ds_dump = (uint16_t *)(base + align_up((size_t)(s->batch + 1) * sizeof(int64_t)));
  a.ds_buf = a.ds_dump + 1024;
  a.ds_head_blocks = ds_head_blocks(s);
  a.batch = s->batch;
}

hstu_status_t hstu_attn_bwd(const hstu_dims_t *dims, const float *rab_pos, const float *rab_time,
                            const hstu_jagged_t *seq, const uint16_t *q, const uint16_t *k,
                            const uint16_t *v, int64_t row_stride, const float *d_out,
                            float *dq, float *dk, float *dv, float *d_rab_pos,
                            float *d_rab_time, void *ws, size_t ws_bytes, void *stream) {
  hstu_status_t st;
  if ((st = check_attn_dims(dims)) != HSTU_OK) return st;
  if ((d_rab_pos != nullptr && rab_pos == nullptr) || (d_rab_time != nullptr && rab_time == nullptr))
    return HSTU_ERR_INVALID_ARG;
  if (!aligned16(d_rab_pos) || !aligned16(d_rab_time)) return HSTU_ERR_INVALID_ARG;
  if ((st = check_seq(seq)) != HSTU_OK) return st;
  const int64_t hq = (int64_t)dims->num_heads * dims->dqk;
  if (seq->total_tokens > 0 && (q == nullptr || k == nullptr || v == nullptr ||
                                d_out == nullptr || dq == nullptr || dk == nullptr ||
                                dv == nullptr))
    return HSTU_ERR_INVALID_ARG;
  if (row_stride < hq || row_stride % 8 != 0) return HSTU_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(d_out) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv))
    return HSTU_ERR_INVALID_ARG;
  const int rab_rows = dims->rab_heads == dims->num_heads && dims->num_heads > 1 ? dims->num_heads : 1;
  if (seq->total_tokens > 0) {  // three distinct outputs, none of them an input
    const void *outs[3] = {dq, dk, dv};
    const void *ins[4] = {q, k, v, d_out};
    for (int i = 0; i < 3; ++i) {
      for (int j = i + 1; j < 3; ++j)
        if (outs[i] == outs[j]) return HSTU_ERR_INVALID_ARG;
      for (const void *in : ins)
        if (outs[i] == in) return HSTU_ERR_INVALID_ARG;
    }
  }
  if (seq->batch == 0 || seq->total_tokens == 0) {  // no pair: the table gradients are zero
    hipError_t e = launch_fill_zero(d_rab_pos, (int64_t)rab_rows * dims->pos_buckets, (hipStream_t)stream);
    if (e == hipSuccess)
      e = launch_fill_zero(d_rab_time, (int64_t)rab_rows * dims->time_buckets, (hipStream_t)stream);
    return e == hipSuccess ? HSTU_OK : hip_fail(e);
  }
  if ((st = check_ws(ws, ws_bytes, attn_bwd_ws_bytes(dims, seq))) != HSTU_OK) return st;
  if (attn_block_m(seq->max_seq_len) != 128) return HSTU_ERR_UNSUPPORTED;  // the kernels' tile
  if (!rows_addressable(seq->max_seq_len, row_stride)) return HSTU_ERR_UNSUPPORTED;

  LayerWs lw{};
  carve_attn((char *)ws, seq, nullptr, lw);
  char *tail = (char *)ws + attn_ws_bytes(seq, nullptr);
  AttnBwdArgs a{};
  {
    const size_t base = attn_bwd_ws_bytes(dims, seq);
    attach_ds(a, dims, seq, (char *)ws + base, ws_bytes - base);
  }
  a.d_h = (uint16_t *)tail;
  a.d_max = (uint32_t *)(tail + align_up((size_t)seq->total_tokens * hq * sizeof(uint16_t)));
  if (d_rab_pos != nullptr || d_rab_time != nullptr) {
    a.rab_part = (float *)(tail + align_up((size_t)seq->total_tokens * hq * sizeof(uint16_t)) + kAlign);
    a.rab_cap = attn_work_capacity(seq->batch, seq->total_tokens);
    a.d_rab_pos = d_rab_pos;
    a.d_rab_time = d_rab_time;
  }
  const bool use_time = rab_time != nullptr && seq->timestamps != nullptr;
  a.stat = use_time ? lw.kstat : nullptr;
  a.offsets = seq->seq_offsets;
  a.ts = seq->timestamps;
  a.q = q;
  a.k = k;
  a.v = v;
  a.stride = row_stride;
  a.d_out = d_out;
  a.d_stride = hq;
  a.rab_pos = rab_pos;
  a.rab_time = rab_time;
  a.pos_buckets = dims->pos_buckets;
  a.time_buckets = dims->time_buckets;
  a.rab_per_head = dims->rab_heads == dims->num_heads && dims->num_heads > 1;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.g_stride = hq;
  a.work = lw.work;
  a.n_work = lw.n_work;
  a.num_heads = dims->num_heads;
  hipStream_t sst = (hipStream_t)stream;
  hipError_t e = launch_schedule(seq->seq_offsets, nullptr, seq->batch, 0, seq->max_seq_len, 0,
                                 lw.work, lw.n_work, sst);
  if (e != hipSuccess) return hip_fail(e);
  if (use_time) {
    e = launch_block_stats(seq->timestamps, seq->seq_offsets, seq->batch, seq->max_seq_len,
                           lw.kstat, sst);
    if (e != hipSuccess) return hip_fail(e);
  }
  const int64_t cap = attn_work_capacity(seq->batch, seq->total_tokens);
  e = launch_attention_bwd(a, dims->dqk, cap, seq->total_tokens, sst);
  if (e != hipSuccess) return hip_fail(e);
  return HSTU_OK;
}

// ------------------------------------------------------------------------------------
// Layer backward
// ------------------------------------------------------------------------------------
namespace {

constexpr int kColsumParts = 1024;

struct LayerBwdWs {
  uint16_t *z, *uvqk, *d_h, *dy16, *g16, *dz;
  float *o, *dg, *d_o, *part_cols, *part_gamma, *part_beta, *rab_part, *tn_part;
  uint32_t *d_max;
  char *attn;
};

// z, U|V|Q|K (fp16 [T][n1]), O, dG, dO (fp32 [T][hdv]), the attention scratch, the
// scaled fp16 dO and its maximum, dY and G in bf16, dZ (bf16 [T][n1]), the partial
// column sums of the bias and LayerNorm gradients, and the split partials of the two
// weight-gradient products (dw2 = dY^T G, dw1 = dZ^T X; one region, used in turn).
size_t layer_bwd_ws(const hstu_dims_t *d, const hstu_jagged_t *s, LayerBwdWs *w) {
  const size_t T = (size_t)s->total_tokens, hdv = (size_t)d->num_heads * d->dv;
  const size_t n1 = 2 * (size_t)d->num_heads * (d->dqk + d->dv), dm = (size_t)d->d_model;
  const size_t waves = (size_t)norm_gate_bwd_waves((int)T);
  const size_t tn = std::max(gemm_tn_partial_bytes((int)dm, (int)hdv, (int)T),
                             gemm_tn_partial_bytes((int)n1, (int)dm, (int)T));
  const size_t sizes[] = {T * n1 * 2, T * n1 * 2, T * hdv * 4, attn_ws_bytes(s, nullptr),
                          T * hdv * 2, kAlign, T * dm * 2, T * hdv * 4, T * hdv * 4,
                          T * hdv * 2, T * n1 * 2, kColsumParts * (n1 > dm ? n1 : dm) * 4,
                          waves * hdv * 4, waves * hdv * 4, rab_part_bytes(d, s), tn};
  size_t off[sizeof(sizes) / sizeof(sizes[0]) + 1] = {0};
  for (size_t i = 0; i < sizeof(sizes) / sizeof(sizes[0]); ++i) off[i + 1] = off[i] + align_up(sizes[i]);
  if (w != nullptr) {
    char *b = (char *)w->attn;  // the base is passed in through attn
    w->z = (uint16_t *)(b + off[0]);
    w->uvqk = (uint16_t *)(b + off[1]);
    w->o = (float *)(b + off[2]);
    w->attn = b + off[3];
    w->d_h = (uint16_t *)(b + off[4]);
    w->d_max = (uint32_t *)(b + off[5]);
    w->dy16 = (uint16_t *)(b + off[6]);
    w->dg = (float *)(b + off[7]);
    w->d_o = (float *)(b + off[8]);
    w->g16 = (uint16_t *)(b + off[9]);
    w->dz = (uint16_t *)(b + off[10]);
    w->part_cols = (float *)(b + off[11]);
    w->part_gamma = (float *)(b + off[12]);
    w->part_beta = (float *)(b + off[13]);
    w->rab_part = (float *)(b + off[14]);
    w->tn_part = (float *)(b + off[15]);
  }
  return off[sizeof(sizes) / sizeof(sizes[0])];
}

}  // namespace

size_t hstu_layer_bwd_workspace_bytes(const hstu_dims_t *dims, const hstu_jagged_t *seq) {
  if (check_dims(dims) != HSTU_OK || check_seq(seq) != HSTU_OK) return 0;
  return layer_bwd_ws(dims, seq, nullptr) + ds_bytes(dims, seq);
}

size_t hstu_layer_bwd_min_workspace_bytes(const hstu_dims_t *dims, const hstu_jagged_t *seq) {
  if (check_dims(dims) != HSTU_OK || check_seq(seq) != HSTU_OK) return 0;
  return layer_bwd_ws(dims, seq, nullptr);
}

}  // extern "C"

namespace {

// Saved forward activations (hstu_layer_fwd_train): U|V|Q|K and the attention's
// standardised output with its statistics; all nullptr to recompute them from x.
struct SavedActs {
  const uint16_t *uvqk, *cn;
  const float2 *stats;
};

hstu_status_t layer_bwd(const hstu_dims_t *dims, const hstu_weights_t *w,
                        const hstu_jagged_t *seq, const uint16_t *x, const float *d_y,
                        float *d_x, const hstu_layer_grads_t *grads, void *ws,
                        size_t ws_bytes, void *stream, const SavedActs &sv) {
  hstu_status_t st;
  if ((st = check_dims(dims)) != HSTU_OK) return st;
  if ((st = check_seq(seq)) != HSTU_OK) return st;
  if ((st = check_weights(w)) != HSTU_OK) return st;
  if (grads == nullptr || grads->w1 == nullptr || grads->w2 == nullptr) return HSTU_ERR_INVALID_ARG;
  if ((grads->rab_pos != nullptr && w->rab_pos == nullptr) ||
      (grads->rab_time != nullptr && w->rab_time == nullptr))
    return HSTU_ERR_INVALID_ARG;
  if ((grads->ln_gamma != nullptr && w->ln_gamma == nullptr) ||
      (grads->ln_beta != nullptr && w->ln_beta == nullptr))
    return HSTU_ERR_INVALID_ARG;
  const void *gr[] = {grads->w1, grads->b1, grads->w2, grads->b2, grads->ln_gamma, grads->ln_beta,
                      grads->rab_pos, grads->rab_time};
  for (const void *g : gr)
    if (!aligned16(g)) return HSTU_ERR_INVALID_ARG;
  if (seq->total_tokens > 0 && (x == nullptr || d_y == nullptr || d_x == nullptr))
    return HSTU_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(d_y) || !aligned16(d_x)) return HSTU_ERR_INVALID_ARG;
  if (seq->total_tokens > 0 && ((const void *)d_x == (const void *)x ||
                                (const void *)d_x == (const void *)d_y))
    return HSTU_ERR_INVALID_ARG;
  for (const void *g : gr)
    if (g != nullptr && g == (const void *)d_x) return HSTU_ERR_INVALID_ARG;
  const bool saved = sv.uvqk != nullptr;
  if (saved) {
    const void *sp[] = {sv.uvqk, sv.cn, sv.stats};
    for (const void *q : sp) {
      if (!aligned16(q) || q == (const void *)d_x) return HSTU_ERR_INVALID_ARG;
      for (const void *g : gr)
        if (g != nullptr && g == q) return HSTU_ERR_INVALID_ARG;
    }
  }
  hipStream_t sst = (hipStream_t)stream;
  const int T = seq->total_tokens;
  const int dm = dims->d_model, hdv = dims->num_heads * dims->dv, hqk = dims->num_heads * dims->dqk;
  const int n1 = 2 * (hdv + hqk);
  const int rab_rows = dims->rab_heads == dims->num_heads && dims->num_heads > 1 ? dims->num_heads : 1;
  if (seq->batch == 0 || T == 0) {  // no token: every formed gradient is zero
    hipError_t e = hipSuccess;
    const std::pair<float *, int64_t> z[] = {{grads->w1, (int64_t)n1 * dm}, {grads->b1, n1},
                                             {grads->w2, (int64_t)dm * hdv}, {grads->b2, dm},
                                             {grads->ln_gamma, hdv}, {grads->ln_beta, hdv},
                                             {grads->rab_pos, (int64_t)rab_rows * dims->pos_buckets},
                                             {grads->rab_time, (int64_t)rab_rows * dims->time_buckets}};
    for (const auto &p : z)
      if (e == hipSuccess) e = launch_fill_zero(p.first, p.second, sst);
    return e == hipSuccess ? HSTU_OK : hip_fail(e);
  }
  if ((st = check_ws(ws, ws_bytes, layer_bwd_ws(dims, seq, nullptr))) != HSTU_OK) return st;
  if (!rows_addressable(seq->max_seq_len, n1)) return HSTU_ERR_UNSUPPORTED;
  if (attn_block_m(seq->max_seq_len) != 128) return HSTU_ERR_UNSUPPORTED;

  LayerBwdWs b{};
  b.attn = (char *)ws;
  layer_bwd_ws(dims, seq, &b);
  LayerWs lw{};
  carve_attn(b.attn, seq, nullptr, lw);
  lw.o = b.o;
  const uint16_t *uvqk = saved ? sv.uvqk : b.uvqk;
  const uint16_t *q = uvqk + 2 * hdv, *k = uvqk + 2 * hdv + hqk, *v = uvqk + hdv;
  AttnArgs aa = attn_args(dims, w->rab_pos, w->rab_time, seq, q, k, v, n1, b.o, lw);
  if ((st = run_setup(seq, aa, lw, nullptr, false, sst)) != HSTU_OK) return st;
  hipError_t e;
#define HSTU_TRY(call)            \
  do {                            \
    e = (call);                   \
    if (e != hipSuccess) return hip_fail(e); \
  } while (0)
  // forward pieces: Z (for SiLU'), then U|V|Q|K = SiLU(Z) and the attention output O
  // unless the forward saved them
  HSTU_TRY(launch_gemm(x, w->w1, w->b1, b.z, T, n1, dm, ACT_NONE, OUT_F16, sst));
  const int64_t cap = attn_work_capacity(seq->batch, T);
  if (!saved) {
    HSTU_TRY(launch_silu_f16(b.z, b.uvqk, (int64_t)T * n1, sst));
    HSTU_TRY(launch_attention(aa, dims->dqk, seq->max_seq_len, cap, sst));
  }
  // f2: dG = dY w2, then the gate and LayerNorm backward, then dw2 = dY^T G, db2
  HSTU_TRY(launch_cast_bf16(d_y, b.dy16, (int64_t)T * dm, sst));
  HSTU_TRY(launch_gemm_nn_f32(b.dy16, dm, w->w2, hdv, b.dg, T, hdv, dm, sst));
  NormGateBwdArgs ng{};
  ng.o = saved ? nullptr : b.o;
  ng.cn = sv.cn;
  ng.stats = sv.stats;
  ng.dv = dims->dv;
  ng.dg = b.dg;
  ng.u = uvqk;
  ng.zu = b.z;
  ng.u_stride = n1;
  ng.gamma = w->ln_gamma;
  ng.beta = w->ln_beta;
  ng.eps = dims->ln_eps;
  ng.g = b.g16;
  ng.dzu = b.dz;
  ng.dz_stride = n1;
  ng.d_o = b.d_o;
  ng.part_gamma = grads->ln_gamma != nullptr ? b.part_gamma : nullptr;
  ng.part_beta = grads->ln_beta != nullptr ? b.part_beta : nullptr;
  ng.T = T;
  ng.hdv = hdv;
  HSTU_TRY(launch_norm_gate_bwd(ng, sst));
  HSTU_TRY(launch_gemm_tn_f32(b.dy16, dm, b.g16, hdv, grads->w2, dm, hdv, T, b.tn_part, sst));
  if (grads->b2 != nullptr)
    HSTU_TRY(launch_colsum(d_y, false, T, dm, dm, b.part_cols, kColsumParts, grads->b2, sst));
  const int waves = norm_gate_bwd_waves(T);
  if (grads->ln_gamma != nullptr) HSTU_TRY(launch_sum_parts(b.part_gamma, waves, hdv, grads->ln_gamma, sst));
  if (grads->ln_beta != nullptr) HSTU_TRY(launch_sum_parts(b.part_beta, waves, hdv, grads->ln_beta, sst));
  // attention: dZ of the V, Q, K columns
  AttnBwdArgs a{};
  a.offsets = seq->seq_offsets;
  a.ts = seq->timestamps;
  a.q = q;
  a.k = k;
  a.v = v;
  a.stride = n1;
  a.d_out = b.d_o;
  a.d_stride = hdv;
  a.d_h = b.d_h;
  a.d_max = b.d_max;
  a.stat = (w->rab_time != nullptr && seq->timestamps != nullptr) ? lw.kstat : nullptr;
  a.rab_pos = w->rab_pos;
  a.rab_time = w->rab_time;
  a.pos_buckets = dims->pos_buckets;
  a.time_buckets = dims->time_buckets;
  a.rab_per_head = dims->rab_heads == dims->num_heads && dims->num_heads > 1;
  a.work = lw.work;
  a.n_work = lw.n_work;
  a.num_heads = dims->num_heads;
  a.z = b.z;
  a.dz = b.dz;
  a.z_stride = n1;
  a.zq_off = 2 * hdv;
  a.zk_off = 2 * hdv + hqk;
  a.zv_off = hdv;
  {
    const size_t base = layer_bwd_ws(dims, seq, nullptr);
    attach_ds(a, dims, seq, (char *)ws + base, ws_bytes - base);
  }
  if (grads->rab_pos != nullptr || grads->rab_time != nullptr) {
    a.rab_part = b.rab_part;
    a.rab_cap = cap;
    a.d_rab_pos = grads->rab_pos;
    a.d_rab_time = grads->rab_time;
  }
  HSTU_TRY(launch_attention_bwd(a, dims->dqk, cap, T, sst));
  // f1: dX = dZ w1, dw1 = dZ^T X, db1
  HSTU_TRY(launch_gemm_nn_f32(b.dz, n1, w->w1, dm, d_x, T, dm, n1, sst));
  HSTU_TRY(launch_gemm_tn_f32(b.dz, n1, x, dm, grads->w1, n1, dm, T, b.tn_part, sst));
  if (grads->b1 != nullptr)
    HSTU_TRY(launch_colsum(b.dz, true, T, n1, n1, b.part_cols, kColsumParts, grads->b1, sst));
#undef HSTU_TRY
  return HSTU_OK;
}

}  // namespace

extern "C" {

hstu_status_t hstu_layer_bwd(const hstu_dims_t *dims, const hstu_weights_t *w,
                             const hstu_jagged_t *seq, const uint16_t *x, const float *d_y,
                             float *d_x, const hstu_layer_grads_t *grads, void *ws,
                             size_t ws_bytes, void *stream) {
  return layer_bwd(dims, w, seq, x, d_y, d_x, grads, ws, ws_bytes, stream, SavedActs{});
}

hstu_status_t hstu_layer_bwd_saved(const hstu_dims_t *dims, const hstu_weights_t *w,
                                   const hstu_jagged_t *seq, const uint16_t *x,
                                   const uint16_t *uvqk, const uint16_t *cn, const float *stats,
                                   const float *d_y, float *d_x, const hstu_layer_grads_t *grads,
                                   void *ws, size_t ws_bytes, void *stream) {
  if (seq != nullptr && seq->total_tokens > 0 && (uvqk == nullptr || cn == nullptr || stats == nullptr))
    return HSTU_ERR_INVALID_ARG;
  if (uvqk == nullptr) {  // empty batch: no activation to read, the ordinary path zeroes
    return layer_bwd(dims, w, seq, x, d_y, d_x, grads, ws, ws_bytes, stream, SavedActs{});
  }
  return layer_bwd(dims, w, seq, x, d_y, d_x, grads, ws, ws_bytes, stream,
                   SavedActs{uvqk, cn, reinterpret_cast<const float2 *>(stats)});
}

}  // extern "C"

namespace {

constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;

}  // namespace

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

// Clock samples of the attention kernel while profiling (kClockSlots pairs per GPU).
static __device__ __align__(256) uint64_t clk_samples[2 * kClockSlots];

namespace {

std::mutex g_clk_mu;
uint64_t *g_clk_ptr[64] = {};

// This device's copy of clk_samples (its address taken once per device), or nullptr.
uint64_t *clock_samples() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lk(g_clk_mu);
  if (g_clk_ptr[dev] == nullptr) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(clk_samples)) != hipSuccess) return nullptr;
    g_clk_ptr[dev] = (uint64_t *)p;
  }
  return g_clk_ptr[dev];
}

}  // namespace

namespace {

// Host checks of an attention call; on success max_prefix is the prefix's longest length.
hstu_status_t check_attn_call(const hstu_dims_t *dims, const hstu_jagged_t *seq,
                              const uint16_t *q, const uint16_t *k, const uint16_t *v,
                              int64_t row_stride, const hstu_prefix_t *prefix, hstu_mask_t mask,
                              const float *out, int &max_prefix) {
  hstu_status_t st;
  if ((st = check_attn_dims(dims)) != HSTU_OK) return st;
  if ((st = check_seq(seq)) != HSTU_OK) return st;
  if (mask != HSTU_MASK_CAUSAL && mask != HSTU_MASK_SELF_ONLY) return HSTU_ERR_INVALID_ARG;
  const int64_t hq = (int64_t)dims->num_heads * dims->dqk;
  if (seq->total_tokens > 0 && (q == nullptr || k == nullptr || v == nullptr || out == nullptr))
    return HSTU_ERR_INVALID_ARG;
  if (row_stride < hq || row_stride % 8 != 0) return HSTU_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return HSTU_ERR_INVALID_ARG;
  max_prefix = 0;
  if (prefix != nullptr) {
    if ((st = check_seq(prefix->seq)) != HSTU_OK) return st;
    if (prefix->seq->batch != seq->batch) return HSTU_ERR_INVALID_ARG;
    if (prefix->seq->total_tokens > 0 && (prefix->k == nullptr || prefix->v == nullptr))
      return HSTU_ERR_INVALID_ARG;
    if (prefix->row_stride < hq || prefix->row_stride % 8 != 0) return HSTU_ERR_INVALID_ARG;
    if (prefix->row_stride != row_stride) return HSTU_ERR_UNSUPPORTED;  // one row pitch
    if (!aligned16(prefix->k) || !aligned16(prefix->v)) return HSTU_ERR_INVALID_ARG;
    if ((prefix->seq->timestamps == nullptr) != (seq->timestamps == nullptr))
      return HSTU_ERR_INVALID_ARG;
    max_prefix = prefix->seq->max_seq_len;
  }
  if (seq->batch == 0 || seq->total_tokens == 0) return HSTU_OK;
  if (!rows_addressable(seq->max_seq_len, row_stride) ||
      (prefix != nullptr && !rows_addressable(prefix->seq->max_seq_len, prefix->row_stride)))
    return HSTU_ERR_UNSUPPORTED;
  return HSTU_OK;
}

// Schedule, key-block timestamp ranges and the attention kernel of a checked call, with
// their scratch carved from ws (attn_ws_bytes(seq, prefix seq) bytes, 256-byte aligned).
// `profile` brackets the launches with the optional timing events.
hstu_status_t launch_attn_call(const hstu_dims_t *dims, const float *rab_pos,
                               const float *rab_time, const hstu_jagged_t *seq, const uint16_t *q,
                               const uint16_t *k, const uint16_t *v, int64_t row_stride,
                               const hstu_prefix_t *prefix, hstu_mask_t mask, float *out,
                               int max_prefix, char *ws, hipStream_t sst, bool profile) {
  const hstu_jagged_t *pre_seq = prefix != nullptr ? prefix->seq : nullptr;
  LayerWs lw{};
  carve_attn(ws, seq, pre_seq, lw);
  AttnArgs aa = attn_args(dims, rab_pos, rab_time, seq, q, k, v, row_stride, out, lw);
  aa.mask = mask == HSTU_MASK_CAUSAL ? 0 : 1;
  if (prefix != nullptr) {
    aa.p_offsets = prefix->seq->seq_offsets;
    aa.p_ts = prefix->seq->timestamps;
    aa.pk = prefix->k;
    aa.pv = prefix->v;
    aa.p_stride = prefix->row_stride;
  }
  auto maybe_timed = [&](int id, auto &&fn) { return profile ? timed(id, sst, fn) : fn(); };
  hipError_t e = maybe_timed(0, [&] {
    return launch_schedule(seq->seq_offsets, aa.p_offsets, seq->batch, aa.mask, seq->max_seq_len,
                           max_prefix, lw.work, lw.n_work, sst);
  });
  if (e != hipSuccess) return hip_fail(e);
  e = maybe_timed(0, [&] { return launch_stats(aa, seq, pre_seq, sst); });
  if (e != hipSuccess) return hip_fail(e);
  const int64_t cap = attn_work_capacity(seq->batch, seq->total_tokens);
  e = maybe_timed(2, [&] { return launch_attention(aa, dims->dqk, seq->max_seq_len, cap, sst); });
  if (e != hipSuccess) return hip_fail(e);
  return HSTU_OK;
}

// ------------------------------------------------------------------------------------
// Scratch of hstu_attn_fwd_noalloc: a static device array (one copy per GPU, held until
// the process ends) instead of a caller workspace.  In host code `scratch` only names the
// symbol; its device address on the current GPU comes from hipGetSymbolAddress, taken
// once per device and cached here, and only that address is ever handed to a kernel.
// ------------------------------------------------------------------------------------
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of the current GPU's scratch array, looked up on first use.
hstu_status_t scratch_on_current_device(char **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= kMaxDevices) return HSTU_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e);
    if (ptr == nullptr) return hip_fail(hipErrorInvalidSymbol);
    g_scratch_ptr[dev] = ptr;
  }
  *out = (char *)g_scratch_ptr[dev];
  return HSTU_OK;
}

}  // namespace

extern "C" {

hstu_status_t hstu_attn_fwd(const hstu_dims_t *dims, const float *rab_pos, const float *rab_time,
                            const hstu_jagged_t *seq, const uint16_t *q, const uint16_t *k,
                            const uint16_t *v, int64_t row_stride, const hstu_prefix_t *prefix,
                            hstu_mask_t mask, float *out, void *ws, size_t ws_bytes,
                            void *stream) {
  int max_prefix = 0;
  hstu_status_t st = check_attn_call(dims, seq, q, k, v, row_stride, prefix, mask, out, max_prefix);
  if (st != HSTU_OK) return st;
  if (seq->batch == 0 || seq->total_tokens == 0) return HSTU_OK;
  const hstu_jagged_t *pre_seq = prefix != nullptr ? prefix->seq : nullptr;
  if ((st = check_ws(ws, ws_bytes, attn_ws_bytes(seq, pre_seq))) != HSTU_OK) return st;
  return launch_attn_call(dims, rab_pos, rab_time, seq, q, k, v, row_stride, prefix, mask, out,
                          max_prefix, (char *)ws, (hipStream_t)stream, true);
}

size_t hstu_attn_noalloc_max_scratch_bytes(void) { return kNoAllocScratchBytes; }

hstu_status_t hstu_attn_fwd_noalloc(const hstu_dims_t *dims, const float *rab_pos,
                                    const float *rab_time, const hstu_jagged_t *seq,
                                    const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                    int64_t row_stride, const hstu_prefix_t *prefix,
                                    hstu_mask_t mask, float *out, void *stream) {
  int max_prefix = 0;
  hstu_status_t st = check_attn_call(dims, seq, q, k, v, row_stride, prefix, mask, out, max_prefix);
  if (st != HSTU_OK) return st;
  if (seq->batch == 0 || seq->total_tokens == 0) return HSTU_OK;
  const hstu_jagged_t *pre_seq = prefix != nullptr ? prefix->seq : nullptr;
  if (attn_ws_bytes(seq, pre_seq) > kNoAllocScratchBytes) return HSTU_ERR_WORKSPACE;
  char *ws = nullptr;
  if ((st = scratch_on_current_device(&ws)) != HSTU_OK) return st;
  return launch_attn_call(dims, rab_pos, rab_time, seq, q, k, v, row_stride, prefix, mask, out,
                          max_prefix, ws, (hipStream_t)stream, false);
}

size_t hstu_sl_workspace_bytes(const hstu_jagged_t *raw) {
  if (check_seq(raw) != HSTU_OK) return 0;
  return align_up((size_t)raw->batch * sizeof(int32_t) + 1);
}

hstu_status_t hstu_stochastic_length(const hstu_jagged_t *raw, const double *u_keep,
                                     const uint32_t *keys, int32_t n_target, double alpha,
                                     int32_t *kept, int32_t *new_offsets, int32_t *new_ts,
                                     const uint16_t *x_raw, uint16_t *x_out, int64_t row_elems,
                                     void *ws, size_t ws_bytes, void *stream) {
  hstu_status_t st;
  if ((st = check_seq(raw)) != HSTU_OK) return st;
  if (n_target < 1 || !(alpha > 0.0) || !std::isfinite(alpha)) return HSTU_ERR_INVALID_ARG;
  // L = floor(N^(alpha/2)); the whole-user threshold numerator N^alpha, both in fp64
  const double l_real = std::floor(std::pow((double)n_target, alpha / 2.0));
  const double thr_num = std::pow((double)n_target, alpha);
  if (!(l_real >= 1.0) || l_real > 2147483647.0 || !std::isfinite(thr_num))
    return HSTU_ERR_INVALID_ARG;
  if (new_offsets == nullptr || (raw->batch > 0 && u_keep == nullptr)) return HSTU_ERR_INVALID_ARG;
  if (raw->total_tokens > 0 && (keys == nullptr || kept == nullptr)) return HSTU_ERR_INVALID_ARG;
  if (new_ts != nullptr && raw->timestamps == nullptr && raw->total_tokens > 0)
    return HSTU_ERR_INVALID_ARG;
  if ((x_raw == nullptr) != (x_out == nullptr)) return HSTU_ERR_INVALID_ARG;
  if (x_raw != nullptr) {
    if (row_elems <= 0 || row_elems % 8 != 0) return HSTU_ERR_INVALID_ARG;
    if (!aligned16(x_raw) || !aligned16(x_out)) return HSTU_ERR_INVALID_ARG;
    if ((const void *)x_raw == (const void *)x_out) return HSTU_ERR_INVALID_ARG;
  }
  // no users: only new_offsets[0] = 0 is written (by the lengths kernel), no workspace
  if (raw->batch > 0 && (st = check_ws(ws, ws_bytes, hstu_sl_workspace_bytes(raw))) != HSTU_OK)
    return st;
  hipError_t e = launch_stochastic_length(raw->seq_offsets, u_keep, keys, raw->batch,
                                          raw->total_tokens, (int)l_real,
                                          thr_num, new_offsets, (int32_t *)ws, raw->timestamps,
                                          kept, new_ts, x_raw, x_out, row_elems, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e);
  return HSTU_OK;
}

hstu_status_t hstu_validate_jagged(const hstu_jagged_t *seq, void *stream) {
  hstu_status_t st;
  if ((st = check_seq(seq)) != HSTU_OK) return st;
  std::vector<int32_t> off((size_t)seq->batch + 1);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(off.data(), seq->seq_offsets, off.size() * sizeof(int32_t),
                                hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e);
  if (off[0] != 0 || off[seq->batch] > seq->total_tokens) return HSTU_ERR_INVALID_ARG;
  for (int b = 0; b < seq->batch; ++b) {
    const int64_t n = (int64_t)off[b + 1] - off[b];
    if (n < 0 || n > seq->max_seq_len) return HSTU_ERR_INVALID_ARG;
  }
  return HSTU_OK;
}

const char *hstu_status_str(hstu_status_t s) {
  switch (s) {
    case HSTU_OK: return "ok";
    case HSTU_ERR_INVALID_ARG: return "invalid argument";
    case HSTU_ERR_UNSUPPORTED: return "unsupported shape";
    case HSTU_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
    case HSTU_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

int hstu_last_hip_error(void) { return g_last_hip_error; }

void hstu_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_mask = on & ((1 << kNumKernels) - 1);
}

void hstu_profile_reset(void) {
  if (uint64_t *p = clock_samples()) (void)hipMemset(p, 0, 2 * kClockSlots * sizeof(uint64_t));
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (auto &r : g_prof_records) {
    g_event_pool.push_back(r.start);
    g_event_pool.push_back(r.stop);
  }
  g_prof_records.clear();
}

hstu_status_t hstu_profile_collect(double *total_ms, int64_t *launches) {
  if (total_ms == nullptr || launches == nullptr) return HSTU_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (int i = 0; i < kNumKernels; ++i) {
    total_ms[i] = 0.0;
    launches[i] = 0;
  }
  for (auto &r : g_prof_records) {
    hipError_t e = hipEventSynchronize(r.stop);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.start, r.stop);
    if (e != hipSuccess) return hip_fail(e);
    total_ms[r.id] += ms;
    launches[r.id] += 1;
  }
  return HSTU_OK;
}

hstu_status_t hstu_profile_clock_ghz(double *ghz) {
  if (ghz == nullptr) return HSTU_ERR_INVALID_ARG;
  *ghz = 0.0;
  uint64_t *p = clock_samples();
  if (p == nullptr) return HSTU_ERR_HIP;
  uint64_t h[2 * kClockSlots];
  hipError_t e = hipMemcpy(h, p, sizeof(h), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e);
  double core = 0.0, real = 0.0;
  for (int i = 0; i < kClockSlots; ++i) {
    core += (double)h[2 * i];
    real += (double)h[2 * i + 1];
  }
  if (real > 0.0) *ghz = core / real * 0.1;  // the real-time counter runs at 100 MHz
  return HSTU_OK;
}

const char *hstu_kernel_name(int id) {
  return (id >= 0 && id < kNumKernels) ? kKernelNames[id] : "unknown";
}

}  // extern "C"
