// Host side of the layer shard: argument validation, carving of the saved-activation
// and workspace buffers, and the launch sequences of forward and backward on the
// caller's stream. Exposes the C ABI declared in include/mt.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "adamw.hpp"
#include "flash_attn.hpp"
#include "gemm.hpp"
#include "mt.h"
#include "rowwise.hpp"

namespace mt {
namespace {

constexpr float kLnEps = 1e-5f;  // LayerNorm epsilon (silent on the pages; common default)

// ------------------------------------------------------------------------- shapes
struct Dims {
  int64_t M, h, heads, at, d, seq, B, tp, hs, qkv, ft;
  bool bf16;
  bool comp;   // MT_BF16_QK: Q and K as hi + lo pairs in the logits
  bool flash;  // fused attention kernels (bf16 path, head dims they support)
  int64_t es;  // bytes per activation element
};

int validate_shape(const mt_shape* s, Dims* out) {
  if (!s) return MT_ERR_INVALID_ARG;
  if (s->h <= 0 || s->heads <= 0 || s->seq <= 0 || s->micro_batch <= 0 || s->tp <= 0) return MT_ERR_INVALID_ARG;
  if (s->shard < 0 || s->shard >= s->tp) return MT_ERR_INVALID_ARG;
  if (s->dtype != MT_BF16 && s->dtype != MT_FP32 && s->dtype != MT_BF16_QK) return MT_ERR_INVALID_ARG;
  if (s->h % s->heads != 0 || s->heads % s->tp != 0) return MT_ERR_INVALID_ARG;
  const int64_t d = s->h / s->heads;
  if (d % 8 != 0 || s->seq % 8 != 0) return MT_ERR_UNSUPPORTED;
  if (s->seq > kSoftmaxMaxSeq) return MT_ERR_UNSUPPORTED;
  if (s->h > kLnMaxH) return MT_ERR_UNSUPPORTED;
  const int64_t M = (int64_t)s->micro_batch * s->seq;
  if (M > (1 << 24)) return MT_ERR_UNSUPPORTED;
  Dims x;
  x.M = M;
  x.h = s->h;
  x.heads = s->heads;
  x.tp = s->tp;
  x.at = s->heads / s->tp;
  x.d = d;
  x.seq = s->seq;
  x.B = s->micro_batch;
  x.hs = x.at * d;
  x.qkv = 3 * x.hs;
  x.ft = 4 * x.h / x.tp;
  x.bf16 = s->dtype != MT_FP32;
  x.comp = s->dtype == MT_BF16_QK;
  x.flash = x.bf16 && flash_supported((int)d);
  x.es = x.bf16 ? 2 : 4;
  *out = x;
  return MT_OK;
}

bool aligned16(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Sub-buffers are carved at 256-byte boundaries; the same code sizes (base == null)
// and carves, so the *_bytes queries always match what the calls use.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <class P = void>
  P* take(size_t bytes) {
    off = (off + 255) & ~size_t(255);
    P* p = base ? reinterpret_cast<P*>(base + off) : nullptr;
    off += bytes;
    return p;
  }
};

struct LayerSaved {
  float *mean1, *rstd1, *mean2, *rstd2;
  float* x2;  // residual stream X + O + b_o, fp32
  void *u, *qkv, *p, *ctx, *v2, *a, *z;
  // fused attention (instead of P): row log-sum-exp [B, a_t, s] and (MT_BF16_QK) the
  // Q, K remainders
  float* lse;
  void* qkv_lo;
};

size_t carve_layer_saved(const Dims& d, void* base, LayerSaved* s) {
  Carver c(base);
  s->mean1 = c.take<float>(d.M * 4);
  s->rstd1 = c.take<float>(d.M * 4);
  s->mean2 = c.take<float>(d.M * 4);
  s->rstd2 = c.take<float>(d.M * 4);
  s->u = c.take(d.M * d.h * d.es);
  s->qkv = c.take(d.M * d.qkv * d.es);
  s->p = d.flash ? nullptr : c.take(d.B * d.at * d.seq * d.seq * d.es);
  s->lse = d.flash ? c.take<float>(d.B * d.at * d.seq * 4) : nullptr;
  s->qkv_lo = d.flash && d.comp ? c.take(d.M * d.qkv * 2) : nullptr;
  s->ctx = c.take(d.M * d.hs * d.es);
  s->x2 = c.take<float>(d.M * d.h * 4);
  s->v2 = c.take(d.M * d.h * d.es);
  s->a = c.take(d.M * d.ft * d.es);
  s->z = c.take(d.M * d.ft * d.es);
  return c.off;
}

struct LayerFwdWs {
  float* S;      // scores; before them (MT_BF16_QK) the fp32 partials of the QKV projection
  void* o;       // out-projection partial, then FC2 partial
  void* u_lo;    // MT_BF16_QK: rounding remainder of U
  void* qkv_lo;  // MT_BF16_QK, unfused attention: rounding remainders of Q and K (QKV layout)
};

size_t carve_layer_fwd_ws(const Dims& d, void* base, LayerFwdWs* w) {
  Carver c(base);
  const int64_t qkv_partials = d.comp ? d.M * (d.qkv + 2 * d.hs) : 0;
  const int64_t scores = d.flash ? 0 : d.B * d.at * d.seq * d.seq;
  w->S = c.take<float>(std::max<int64_t>(scores, qkv_partials) * 4);
  w->o = c.take(d.M * d.h * d.es);
  w->u_lo = d.comp ? c.take(d.M * d.h * 2) : nullptr;
  w->qkv_lo = d.comp && !d.flash ? c.take(d.M * d.qkv * 2) : nullptr;  // saved with fused attention
  return c.off;
}

struct LayerBwdWs {
  void *da, *dv2, *dx2, *dctx, *ds, *dqkv;
  float *D, *part;
  float* spart;  // k-slice partials of a split input or weight gradient (bf16 path)
};

GemmArgs plain(const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc, int64_t M, int64_t N,
               int64_t K);

// fp32 k-slice partials of the largest split GEMM of the layer's backward pairs that
// take them (FC1, out-projection, QKV; 0 if none splits): input gradient dg [M, N] over
// K, weight gradient [K, N] over the M tokens.
int64_t dgrad_split_floats(const Dims& d) {
  if (!d.bf16) return 0;
  const int64_t nk[3][2] = {{d.h, d.ft}, {d.hs, d.h}, {d.h, d.qkv}};
  int64_t n = 0;
  for (const auto& p : nk) {
    const GemmArgs dg = plain(nullptr, p[1], nullptr, p[0], nullptr, p[0], d.M, p[0], p[1]);
    const GemmArgs wg = plain(nullptr, p[1], nullptr, p[0], nullptr, p[0], p[1], p[0], d.M);
    n = std::max<int64_t>(n, gemm_pair_split_floats(dg, EPI_STORE, wg));
  }
  return n;
}

size_t colsum_floats(const Dims& d) {
  size_t n = colsum_partial_floats((int)d.M, (int)d.h, 1);
  n = std::max(n, colsum_partial_floats((int)d.M, (int)d.ft, 0));
  n = std::max(n, gemm_colsum_floats((int)d.M, (int)d.ft));
  n = std::max(n, colsum_partial_floats((int)d.M, (int)d.qkv, 0));
  if (d.flash) n = std::max(n, (size_t)(flash_dbias_rows((int)d.B, (int)d.seq) * d.qkv));
  if (ln_bwd_sums_supported((int)d.h)) n = std::max(n, ln_bwd_sums_partial_floats((int)d.M, (int)d.h, 4));
  return n;
}

size_t carve_layer_bwd_ws(const Dims& d, void* base, LayerBwdWs* w) {
  Carver c(base);
  w->da = c.take(d.M * d.ft * d.es);
  w->dv2 = c.take(d.M * d.h * d.es);  // dV2 partial, later dU partial
  w->dx2 = c.take(d.M * d.h * d.es);
  w->dctx = c.take(d.M * d.hs * d.es);
  w->ds = d.flash ? nullptr : c.take(d.B * d.at * d.seq * d.seq * d.es);
  w->dqkv = c.take(d.M * d.qkv * d.es);
  w->D = c.take<float>(d.B * d.at * d.seq * 4);
  w->part = c.take<float>(colsum_floats(d) * 4);
  const int64_t sp = dgrad_split_floats(d);
  w->spart = sp ? c.take<float>(sp * 4) : nullptr;
  return c.off;
}

struct MlpSaved {
  void *a, *z;
};
size_t carve_mlp_saved(const Dims& d, void* base, MlpSaved* s) {
  Carver c(base);
  s->a = c.take(d.M * d.ft * d.es);
  s->z = c.take(d.M * d.ft * d.es);
  return c.off;
}
struct MlpWs {
  void* da;
  float* part;
};
size_t carve_mlp_ws(const Dims& d, void* base, MlpWs* w) {
  Carver c(base);
  w->da = c.take(d.M * d.ft * d.es);
  w->part = c.take<float>(std::max(colsum_partial_floats((int)d.M, (int)d.ft, 0), gemm_colsum_floats((int)d.M, (int)d.ft)) * 4);
  return c.off;
}

// ------------------------------------------------------------------------- timing
struct TimingRec {
  std::string label;
  hipEvent_t a, b;
  double flops, bytes;
};

// Timing state (the only state the library keeps). g_timing is read without the lock
// by every launch sequence, so it is atomic; the filter, the records and the event pool
// are only touched under g_tmu.
std::mutex g_tmu;
std::atomic<bool> g_timing{false};
std::string g_filter;
std::vector<TimingRec> g_recs;
std::vector<hipEvent_t> g_free;

// An event from the pool, or a new one (hipEventCreate: only while timing is enabled).
// Called with g_tmu held.
hipEvent_t timing_event() {
  if (!g_free.empty()) {
    hipEvent_t e = g_free.back();
    g_free.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Enqueues one launch (f returns hipError_t), optionally bracketed by timing events.
// With timing off (no_timing), a sequence never touches the timing state, so it
// creates no events.
class Seq {
 public:
  explicit Seq(hipStream_t s, bool no_timing = false) : s_(s), no_timing_(no_timing) {}
  template <class F>
  bool run(const char* label, double flops, double bytes, F&& f) {
    if (err_ != hipSuccess) return false;
    hipEvent_t a = nullptr, b = nullptr;
    bool timed = false;
    if (!no_timing_ && g_timing.load(std::memory_order_acquire)) {
      std::lock_guard<std::mutex> lk(g_tmu);
      if (g_timing.load(std::memory_order_relaxed) &&
          (g_filter.empty() || std::strstr(label, g_filter.c_str()) != nullptr)) {
        a = timing_event();
        b = timing_event();
        timed = a && b;
      }
    }
    if (timed && hipEventRecord(a, s_) != hipSuccess) timed = false;
    err_ = f();
    if (timed && hipEventRecord(b, s_) != hipSuccess) timed = false;
    if (a || b) {
      std::lock_guard<std::mutex> lk(g_tmu);
      if (timed) {
        g_recs.push_back({label, a, b, flops, bytes});
      } else {  // a half-acquired or unrecorded pair goes back to the pool
        if (a) g_free.push_back(a);
        if (b) g_free.push_back(b);
      }
    }
    return err_ == hipSuccess;
  }
  int status() const { return err_ == hipSuccess ? MT_OK : MT_ERR_HIP; }
  hipStream_t stream() const { return s_; }

 private:
  hipStream_t s_;
  bool no_timing_;
  hipError_t err_ = hipSuccess;
};

// ------------------------------------------------------------------------- GEMM helpers
GemmArgs plain(const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc, int64_t M, int64_t N,
               int64_t K) {
  GemmArgs g;
  std::memset(&g, 0, sizeof(g));
  g.A = A;
  g.B = B;
  g.C = C;
  g.lda = lda;
  g.ldb = ldb;
  g.ldc = ldc;
  g.M = (int)M;
  g.N = (int)N;
  g.K = (int)K;
  g.zdiv = 1;
  g.alpha = 1.0f;
  g.seg_a[0] = A;
  g.seg_b[0] = B;
  g.nseg = 1;
  g.seg_n = 1 << 30;
  return g;
}

hipError_t gemm(const Dims& d, const GemmArgs& g, bool a_k, bool b_k, int kind, int batch, hipStream_t s) {
  return d.bf16 ? launch_gemm_bf16(g, a_k, b_k, kind, batch, s) : launch_gemm_f32(g, a_k, b_k, kind, batch, s);
}

// Input gradient dg (A k-contiguous, B n-contiguous; epilogue dkind) and weight
// gradient wg (both operands token-strided, fp32 out) of one linear layer: one paired
// launch where the bf16 path supports it, else the two one after the other.
hipError_t gemm_dgrad_wgrad(const Dims& d, const GemmArgs& dg, int dkind, const GemmArgs& wg, hipStream_t s,
                            float* spart = nullptr) {
  if (d.bf16 && spart) {  // a deep input gradient or weight gradient in k slices
    const hipError_t e = launch_gemm_bf16_pair_split(dg, dkind, wg, spart, s);
    if (e != hipErrorNotSupported) return e;
  }
  if (d.bf16) {
    const hipError_t e = launch_gemm_bf16_pair(dg, true, false, dkind, wg, false, false, EPI_STORE_F32, s);
    if (e != hipErrorNotSupported) return e;
  }
  const hipError_t e = gemm(d, wg, false, false, EPI_STORE_F32, 1, s);
  if (e != hipSuccess) return e;
  return gemm(d, dg, true, false, dkind, 1, s);
}

double gflop(double m, double n, double k) { return 2.0 * m * n * k; }

// Per-head attention products over (b, k) pairs: batch z = b * at + k.
struct Attn {
  const Dims& d;
  double causal_pairs() const { return (double)d.seq * (d.seq + 1) / 2.0; }
  double flops() const { return 2.0 * d.d * causal_pairs() * d.B * d.at; }
  // head slice of an [M, ld] activation whose head k starts at column col0 + k*d
  void head_operand(int64_t ld, int64_t& so, int64_t& si) const {
    so = d.seq * ld;
    si = d.d;
  }
};

// Arguments of the fused attention kernels for this shard.
FlashArgs flash_args(const Dims& d, const void* qkv, const void* qkv_lo, void* ctx, float* lse, float scale) {
  FlashArgs a;
  std::memset(&a, 0, sizeof(a));
  a.qkv = qkv;
  a.qkv_lo = qkv_lo;
  a.ctx = ctx;
  a.lse = lse;
  a.ldq = d.qkv;
  a.ldc = d.hs;
  a.batch = (int)d.B;
  a.heads = (int)d.at;
  a.seq = (int)d.seq;
  a.hs = (int)d.hs;
  a.scale = scale;
  return a;
}

// ------------------------------------------------------------------------- forward
// Attention block of the shard (F2-F6): QKV_i = U W_qkv_i^T + b_qkv_i, causal attention
// over the rank's heads, O_i = ctx_i W_o_i^T (the row-parallel partial), from the
// LayerNorm output u [M, h] (and, MT_BF16_QK, its rounding remainder u_lo).
struct AttnBufs {
  void *qkv, *p, *ctx;  // saved: projections, probabilities (unfused), context
  float* lse;           // saved: row log-sum-exp (fused)
  void* qkv_lo_saved;   // saved: Q, K remainders (fused, MT_BF16_QK)
  float* S;             // workspace: scores (unfused) or the QKV partials (MT_BF16_QK)
  void* qkv_lo_ws;      // workspace: Q, K remainders (unfused, MT_BF16_QK)
};

void attn_fwd_part(Seq& q, const Dims& d, const void* u, const void* u_lo, const void* w_qkv, const void* b_qkv,
                   const void* w_o, const AttnBufs& b, void* o, hipStream_t stream) {
  const bool bf = d.bf16;
  const double es = (double)d.es;
  const float scale = 1.0f / std::sqrt((float)d.d);
  const int batch = (int)(d.B * d.at);
  Attn at{d};
  // Q, K remainders (MT_BF16_QK; kept for the backward when fused), else null
  void* qkv_lo = d.flash ? b.qkv_lo_saved : b.qkv_lo_ws;
  (void)bf;
  (void)es;
  // F2 column-parallel QKV projection + bias. MT_BF16_QK: the Q and K columns are formed
  // from U_hi + U_lo (a second K segment) and stored as hi + lo bf16 pairs, so the
  // softmax logits, whose sharp maxima amplify input rounding, see Q and K to ~16 bits.
  q.run("qkv_fwd", gflop(d.M, d.qkv, d.h) + (d.comp ? gflop(d.M, 2 * d.hs, d.h) : 0), 0, [&] {
    GemmArgs g = plain(u, d.h, w_qkv, d.h, b.qkv, d.qkv, d.M, d.qkv, d.h);
    g.vec = b_qkv;
    if (!d.comp) return gemm(d, g, true, true, EPI_BIAS, 1, stream);
    // The Q and K columns take U_hi W^T + U_lo W^T, twice the contraction of the V
    // columns. The two products run as equal-depth problems of one launch into fp32
    // partials (which fills the CUs evenly), and a pass adds them and the bias and
    // splits Q, K into hi + lo.
    float* hi = b.S;
    float* lo = b.S + d.M * d.qkv;
    const GemmArgs ghi = plain(u, d.h, w_qkv, d.h, hi, d.qkv, d.M, d.qkv, d.h);
    const GemmArgs glo = plain(u_lo, d.h, w_qkv, d.h, lo, 2 * d.hs, d.M, 2 * d.hs, d.h);
    const hipError_t e = launch_gemm_bf16_pair(ghi, true, true, EPI_STORE_F32, glo, true, true, EPI_STORE_F32, stream);
    if (e == hipSuccess)
      return launch_qkv_finish(hi, lo, b_qkv, b.qkv, qkv_lo, (int)d.M, (int)d.qkv, (int)(2 * d.hs), stream);
    if (e != hipErrorNotSupported) return e;
    // Operands the paired launch cannot address: one GEMM with a second K segment for
    // the Q and K columns.
    g.seg_a[1] = u_lo;
    g.seg_b[1] = w_qkv;
    g.nseg = 2;
    g.seg_n = (int)(2 * d.hs);
    g.C2 = qkv_lo;
    return gemm(d, g, true, true, EPI_BIAS_SPLIT, 1, stream);
  });
  // F3-F5 causal attention. Fused (bf16, supported head dim): one kernel streams the keys
  // through LDS with an online softmax and keeps S and P on chip; it saves the row
  // log-sum-exp for the backward.
  if (d.flash) {
    q.run("attn_fwd", 2 * at.flops(), 0, [&] {
      FlashArgs fa = flash_args(d, b.qkv, qkv_lo, b.ctx, b.lse, scale);
      return launch_flash_fwd(fa, (int)d.d, stream);
    });
  } else {
    // F3 scores S = Q K^T / sqrt(d), causal tiles only, fp32 (MT_BF16_QK:
    // Q_hi K_hi^T + Q_hi K_lo^T + Q_lo K_hi^T)
    q.run("attn_scores", at.flops() * (d.comp ? 3 : 1), 0, [&] {
      GemmArgs g = plain(b.qkv, d.qkv, static_cast<const char*>(b.qkv) + d.hs * d.es, d.qkv, b.S, d.seq, d.seq,
                         d.seq, d.d);
      if (d.comp) {
        const char* lo = static_cast<const char*>(qkv_lo);
        g.seg_a[1] = b.qkv;
        g.seg_b[1] = lo + d.hs * d.es;
        g.seg_a[2] = lo;
        g.seg_b[2] = static_cast<const char*>(b.qkv) + d.hs * d.es;
        g.nseg = 3;
      }
      at.head_operand(d.qkv, g.a_so, g.a_si);
      at.head_operand(d.qkv, g.b_so, g.b_si);
      g.c_so = d.at * d.seq * d.seq;
      g.c_si = d.seq * d.seq;
      g.zdiv = (int)d.at;
      g.causal = CAUSAL_SKIP_UPPER;
      g.alpha = scale;
      return gemm(d, g, true, true, EPI_STORE_F32, batch, stream);
    });
    // F4 causal softmax -> P
    q.run("softmax_fwd", 0, (double)batch * at.causal_pairs() * (4 + es), [&] {
      return launch_softmax_causal(bf, b.S, b.p, batch, (int)d.seq, stream);
    });
    // F5 ctx = P V (k <= q), heads concatenated in columns
    q.run("attn_ctx", at.flops(), 0, [&] {
      GemmArgs g = plain(b.p, d.seq, static_cast<const char*>(b.qkv) + 2 * d.hs * d.es, d.qkv, b.ctx, d.hs, d.seq,
                         d.d, d.seq);
      g.a_so = d.at * d.seq * d.seq;
      g.a_si = d.seq * d.seq;
      at.head_operand(d.qkv, g.b_so, g.b_si);
      at.head_operand(d.hs, g.c_so, g.c_si);
      g.zdiv = (int)d.at;
      g.causal = CAUSAL_K_LE_M;
      return gemm(d, g, true, false, EPI_STORE, batch, stream);
    });
  }
  // F6 row-parallel out-projection: partial sum O_i (the all-reduce input)
  q.run("out_proj_fwd", gflop(d.M, d.h, d.hs), 0, [&] {
    GemmArgs g = plain(b.ctx, d.hs, w_o, d.hs, o, d.h, d.M, d.h, d.hs);
    return gemm(d, g, true, true, EPI_STORE, 1, stream);
  });
}

AttnBufs attn_bufs(const LayerSaved& sv, const LayerFwdWs& ws) {
  return AttnBufs{sv.qkv, sv.p, sv.ctx, sv.lse, sv.qkv_lo, ws.S, ws.qkv_lo};
}

int layer_fwd_impl(const Dims& d, const mt_layer_weights& w, const void* x, void* out, const LayerSaved& sv,
                   const LayerFwdWs& ws, hipStream_t stream) {
  Seq q(stream);
  const bool bf = d.bf16;
  const double es = (double)d.es;
  const double Mh = (double)d.M * d.h;

  // F1 LayerNorm 1 (MT_BF16_QK: also the rounding remainder U_lo of U)
  q.run("ln1_fwd", 0, Mh * es * (d.comp ? 3 : 2), [&] {
    return launch_ln_fwd(bf, x, w.ln1_g, w.ln1_b, sv.u, ws.u_lo, sv.mean1, sv.rstd1, (int)d.M, (int)d.h, kLnEps,
                         stream);
  });
  attn_fwd_part(q, d, sv.u, ws.u_lo, w.w_qkv, w.b_qkv, w.w_o, attn_bufs(sv, ws), ws.o, stream);
  // F7 X2 = X + AR(O_i) + b_o (AR = identity on one GPU; X2 kept in fp32), V2 = LN2(X2)
  q.run("add_ln2_fwd", 0, Mh * (3 * es + 4), [&] {
    return launch_add_ln_fwd(bf, x, ws.o, w.b_o, w.ln2_g, w.ln2_b, sv.x2, sv.v2, sv.mean2, sv.rstd2, (int)d.M,
                             (int)d.h, kLnEps, stream);
  });
  // F8 column-parallel FC1 with fused bias + GeLU (keeps A and Z)
  q.run("fc1_fwd", gflop(d.M, d.ft, d.h), 0, [&] {
    GemmArgs g = plain(sv.v2, d.h, w.w_fc1, d.h, sv.a, d.ft, d.M, d.ft, d.h);
    g.vec = w.b_fc1;
    g.C2 = sv.z;
    return gemm(d, g, true, true, EPI_BIAS_GELU, 1, stream);
  });
  // F9 row-parallel FC2, partial sum Y_i, and F10 Out = X2 + AR(Y_i) + b_fc2 in its
  // epilogue: with the all-reduce the identity on one GPU, the partial is added to the fp32
  // residual stream and the bias straight from the fp32 accumulators (it is never stored;
  // a tensor-parallel group would store it as the all-reduce's input and add after it, as
  // mt_mlp_fwd and mt_sp_add_fwd do)
  q.run("fc2_fwd", gflop(d.M, d.h, d.ft), 0, [&] {
    GemmArgs g = plain(sv.z, d.ft, w.w_fc2, d.ft, out, d.h, d.M, d.h, d.ft);
    g.vec = w.b_fc2;
    g.aux = sv.x2;
    return gemm(d, g, true, true, EPI_BIAS_RESID, 1, stream);
  });
  return q.status();
}

// ------------------------------------------------------------------------- backward
// Backward of the attention block (B4-B7) given dO [M, h], the gradient of its output:
// dW_o = dO^T ctx, dctx = dO W_o; attention backward; db_qkv, dW_qkv = dQKV^T U and the
// input-gradient partial du = dQKV W_qkv.
struct AttnBwdWs {
  void *dctx, *ds, *dqkv;
  float *D, *part, *spart;
};

void attn_bwd_part(Seq& q, const Dims& d, const void* u, const void* w_qkv, const void* w_o, const AttnBufs& sv,
                   const void* dO, void* du, float* dw_qkv, float* db_qkv, float* dw_o, const AttnBwdWs& ws,
                   hipStream_t stream) {
  const bool bf = d.bf16;
  const double es = (double)d.es;
  const float scale = 1.0f / std::sqrt((float)d.d);
  const int batch = (int)(d.B * d.at);
  const int M = (int)d.M;
  Attn at{d};
  // B4 out-projection: dW_o = dX2^T ctx, dctx = dX2 W_o
  q.run("out_proj_dgrad_wgrad", 2 * gflop(d.M, d.hs, d.h), 0, [&] {
    const GemmArgs dg = plain(dO, d.h, w_o, d.hs, ws.dctx, d.hs, d.M, d.hs, d.h);
    const GemmArgs wg = plain(dO, d.h, sv.ctx, d.hs, dw_o, d.hs, d.h, d.hs, d.M);
    return gemm_dgrad_wgrad(d, dg, EPI_STORE, wg, stream, ws.spart);
  });
  // B5/B6 attention: D = rowsum(dctx * ctx) = rowsum(P * dP); dS = P * (dctx V^T - D)
  q.run("attn_rowdot", 0, 2.0 * d.M * d.hs * es, [&] {
    return launch_attn_rowdot(bf, ws.dctx, sv.ctx, ws.D, (int)d.B, (int)d.seq, (int)d.at, (int)d.d, stream);
  });
  if (d.flash) {
    // B5/B6 fused: P recomputed from Q, K and the saved log-sum-exp; dK, dV per key block
    // and dQ per query block, each summed in one work-group (no atomics), with the column
    // sums of each 64-row block of dQKV for db_qkv.
    q.run("attn_bwd", 4 * at.flops(), 0, [&] {
      FlashArgs fa = flash_args(d, sv.qkv, sv.qkv_lo_saved, nullptr, sv.lse, scale);
      fa.dctx = ws.dctx;
      fa.D = ws.D;
      fa.dqkv = ws.dqkv;
      fa.dbias_part = ws.part;
      return launch_flash_bwd(fa, (int)d.d, stream);
    });
  } else {
    const char* qkv = static_cast<const char*>(sv.qkv);
    char* dqkv = static_cast<char*>(ws.dqkv);
    q.run("attn_dscores", at.flops(), 0, [&] {
      GemmArgs g = plain(ws.dctx, d.hs, qkv + 2 * d.hs * d.es, d.qkv, ws.ds, d.seq, d.seq, d.seq, d.d);
      at.head_operand(d.hs, g.a_so, g.a_si);
      at.head_operand(d.qkv, g.b_so, g.b_si);
      g.c_so = d.at * d.seq * d.seq;
      g.c_si = d.seq * d.seq;
      g.aux = sv.p;
      g.vec = ws.D;
      g.vec_bs = d.seq;
      g.zdiv = (int)d.at;
      g.causal = CAUSAL_SKIP_UPPER;
      return gemm(d, g, true, true, EPI_DSOFTMAX, batch, stream);
    });
    q.run("attn_dv", at.flops(), 0, [&] {  // dV = P^T dctx (q >= j)
      GemmArgs g = plain(sv.p, d.seq, ws.dctx, d.hs, dqkv + 2 * d.hs * d.es, d.qkv, d.seq, d.d, d.seq);
      g.a_so = d.at * d.seq * d.seq;
      g.a_si = d.seq * d.seq;
      at.head_operand(d.hs, g.b_so, g.b_si);
      at.head_operand(d.qkv, g.c_so, g.c_si);
      g.zdiv = (int)d.at;
      g.causal = CAUSAL_K_GE_M;
      return gemm(d, g, false, false, EPI_STORE, batch, stream);
    });
    q.run("attn_dq", at.flops(), 0, [&] {  // dQ = dS K / sqrt(d) (j <= q)
      GemmArgs g = plain(ws.ds, d.seq, qkv + d.hs * d.es, d.qkv, dqkv, d.qkv, d.seq, d.d, d.seq);
      g.a_so = d.at * d.seq * d.seq;
      g.a_si = d.seq * d.seq;
      at.head_operand(d.qkv, g.b_so, g.b_si);
      at.head_operand(d.qkv, g.c_so, g.c_si);
      g.zdiv = (int)d.at;
      g.causal = CAUSAL_K_LE_M;
      g.alpha = scale;
      return gemm(d, g, true, false, EPI_STORE, batch, stream);
    });
    q.run("attn_dk", at.flops(), 0, [&] {  // dK = dS^T Q / sqrt(d) (q >= j)
      GemmArgs g = plain(ws.ds, d.seq, qkv, d.qkv, dqkv + d.hs * d.es, d.qkv, d.seq, d.d, d.seq);
      g.a_so = d.at * d.seq * d.seq;
      g.a_si = d.seq * d.seq;
      at.head_operand(d.qkv, g.b_so, g.b_si);
      at.head_operand(d.qkv, g.c_so, g.c_si);
      g.zdiv = (int)d.at;
      g.causal = CAUSAL_K_GE_M;
      g.alpha = scale;
      return gemm(d, g, false, false, EPI_STORE, batch, stream);
    });
  }
  // B7 QKV: db_qkv, dW_qkv = dQKV^T U, dU = dQKV W_qkv (partial)
  if (d.flash) {  // fixed-order sum of the attention backward's per-block column sums
    const int64_t nrb = flash_dbias_rows((int)d.B, (int)d.seq);
    q.run("db_qkv", 0, nrb * d.qkv * 4.0, [&] { return launch_colsum_final(ws.part, db_qkv, (int)nrb, (int)d.qkv, stream); });
  } else {
    q.run("db_qkv", 0, d.M * d.qkv * es, [&] {
      return launch_colsum(bf, 0, ws.dqkv, false, nullptr, false, nullptr, nullptr, db_qkv, nullptr, ws.part, M,
                           (int)d.qkv, stream);
    });
  }
  q.run("qkv_dgrad_wgrad", 2 * gflop(d.M, d.h, d.qkv), 0, [&] {
    const GemmArgs dg = plain(ws.dqkv, d.qkv, w_qkv, d.h, du, d.h, d.M, d.h, d.qkv);
    const GemmArgs wg = plain(ws.dqkv, d.qkv, u, d.h, dw_qkv, d.h, d.qkv, d.h, d.M);
    return gemm_dgrad_wgrad(d, dg, EPI_STORE, wg, stream, ws.spart);
  });
}

int layer_bwd_impl(const Dims& d, const mt_layer_weights& w, const void* x, const LayerSaved& sv, const void* dout,
                   void* dx, const mt_layer_grads& gr, const LayerBwdWs& ws, hipStream_t stream) {
  Seq q(stream);
  const bool bf = d.bf16;
  const double es = (double)d.es;
  const double Mh = (double)d.M * d.h;
  const int M = (int)d.M;

  // B1 FC2: dW2 = dOut^T Z, dA = (dOut W2) * GeLU'(A); db_fc2 = colsum(dOut) is taken by the
  // LayerNorm-2 pass below (which reads dOut as its residual input) where the fused kernel
  // covers h, else here
  const bool ln_sums = ln_bwd_sums_supported((int)d.h);
  if (!ln_sums)
    q.run("db_fc2", 0, Mh * es, [&] {
      return launch_colsum(bf, 0, dout, false, nullptr, false, nullptr, nullptr, gr.b_fc2, nullptr, ws.part, M,
                           (int)d.h, stream);
    });
  // (bf16: the dgrad epilogue also forms db_fc1's column sums of dA per 128 rows)
  q.run("fc2_dgrad_wgrad", 2 * gflop(d.M, d.ft, d.h), 0, [&] {
    GemmArgs dg = plain(dout, d.h, w.w_fc2, d.ft, ws.da, d.ft, d.M, d.ft, d.h);
    dg.aux = sv.a;
    if (bf) dg.colsum = ws.part;
    const GemmArgs wg = plain(dout, d.h, sv.z, d.ft, gr.w_fc2, d.ft, d.h, d.ft, d.M);
    return gemm_dgrad_wgrad(d, dg, EPI_DGELU, wg, stream);
  });
  // B2 FC1: db_fc1, dW1 = dA^T V2, dV2 = dA W1 (partial)
  q.run("db_fc1", 0, bf ? 4.0 * gemm_colsum_floats(M, (int)d.ft) : d.M * d.ft * es, [&] {
    if (bf) return launch_colsum_final(ws.part, gr.b_fc1, (M + kColsumRows - 1) / kColsumRows, (int)d.ft, stream);
    return launch_colsum(bf, 0, ws.da, false, nullptr, false, nullptr, nullptr, gr.b_fc1, nullptr, ws.part, M,
                         (int)d.ft, stream);
  });
  q.run("fc1_dgrad_wgrad", 2 * gflop(d.M, d.h, d.ft), 0, [&] {
    const GemmArgs dg = plain(ws.da, d.ft, w.w_fc1, d.h, ws.dv2, d.h, d.M, d.h, d.ft);
    const GemmArgs wg = plain(ws.da, d.ft, sv.v2, d.h, gr.w_fc1, d.h, d.ft, d.h, d.M);
    return gemm_dgrad_wgrad(d, dg, EPI_STORE, wg, stream, ws.spart);
  });
  // B3 dX2 = dOut + LN2-backward(AR(dV2)) (the out-projection GEMMs' operand and the
  // residual input of the LayerNorm-1 backward); dgamma2, dbeta2; db_o = colsum(dX2);
  // db_fc2 = colsum(dOut) — in one pass over the rows where the fused kernel covers h (db_o
  // then summed from the unrounded values), else as separate column sums
  if (ln_sums) {
    q.run("ln2_bwd", 0, Mh * (3 * es + 4), [&] {
      return launch_ln_bwd_sums(bf, ws.dv2, sv.x2, true, w.ln2_g, sv.mean2, sv.rstd2, dout, false, ws.dx2, nullptr,
                                ws.part, gr.ln2_g, gr.ln2_b, gr.b_o, gr.b_fc2, M, (int)d.h, stream);
    });
  } else {
    q.run("ln2_bwd", 0, Mh * (3 * es + 4), [&] {
      return launch_ln_bwd(bf, ws.dv2, sv.x2, true, w.ln2_g, sv.mean2, sv.rstd2, dout, false, ws.dx2, nullptr, M,
                           (int)d.h, stream);
    });
    q.run("ln2_param_grads", 0, Mh * (es + 4), [&] {
      return launch_colsum(bf, 1, ws.dv2, false, sv.x2, true, sv.mean2, sv.rstd2, gr.ln2_g, gr.ln2_b, ws.part, M,
                           (int)d.h, stream);
    });
    q.run("db_o", 0, Mh * es, [&] {
      return launch_colsum(bf, 0, ws.dx2, !bf, nullptr, false, nullptr, nullptr, gr.b_o, nullptr, ws.part, M,
                           (int)d.h, stream);
    });
  }
  attn_bwd_part(q, d, sv.u, w.w_qkv, w.w_o, attn_bufs(sv, LayerFwdWs{}), ws.dx2, ws.dv2, gr.w_qkv, gr.b_qkv, gr.w_o,
                AttnBwdWs{ws.dctx, ws.ds, ws.dqkv, ws.D, ws.part, ws.spart}, stream);
  // B8 dX = dX2 + LN1-backward(AR(dU)); dgamma1, dbeta1
  if (ln_sums) {
    q.run("ln1_bwd", 0, Mh * 4 * es, [&] {
      return launch_ln_bwd_sums(bf, ws.dv2, x, false, w.ln1_g, sv.mean1, sv.rstd1, ws.dx2, !bf, dx, nullptr,
                                ws.part, gr.ln1_g, gr.ln1_b, nullptr, nullptr, M, (int)d.h, stream);
    });
  } else {
    q.run("ln1_bwd", 0, Mh * 4 * es, [&] {
      return launch_ln_bwd(bf, ws.dv2, x, false, w.ln1_g, sv.mean1, sv.rstd1, ws.dx2, !bf, dx, nullptr, M,
                           (int)d.h, stream);
    });
    q.run("ln1_param_grads", 0, 2 * Mh * es, [&] {
      return launch_colsum(bf, 1, ws.dv2, false, x, false, sv.mean1, sv.rstd1, gr.ln1_g, gr.ln1_b, ws.part, M,
                           (int)d.h, stream);
    });
  }
  return q.status();
}

// ------------------------------------------------------------------------- MLP block
int mlp_fwd_impl(const Dims& d, const void* x, const void* w1, const void* b1, const void* w2, void* y,
                 const MlpSaved& sv, hipStream_t stream) {
  Seq q(stream);
  q.run("fc1_fwd", gflop(d.M, d.ft, d.h), 0, [&] {
    GemmArgs g = plain(x, d.h, w1, d.h, sv.a, d.ft, d.M, d.ft, d.h);
    g.vec = b1;
    g.C2 = sv.z;
    return gemm(d, g, true, true, EPI_BIAS_GELU, 1, stream);
  });
  q.run("fc2_fwd", gflop(d.M, d.h, d.ft), 0, [&] {
    GemmArgs g = plain(sv.z, d.ft, w2, d.ft, y, d.h, d.M, d.h, d.ft);
    return gemm(d, g, true, true, EPI_STORE, 1, stream);
  });
  return q.status();
}

int mlp_bwd_impl(const Dims& d, const void* x, const void* w1, const void* w2, const MlpSaved& sv, const void* dy,
                 void* dx, float* dw1, float* db1, float* dw2, const MlpWs& ws, hipStream_t stream,
                 bool no_timing = false) {
  Seq q(stream, no_timing);
  q.run("fc2_dgrad_wgrad", 2 * gflop(d.M, d.ft, d.h), 0, [&] {
    GemmArgs dg = plain(dy, d.h, w2, d.ft, ws.da, d.ft, d.M, d.ft, d.h);
    dg.aux = sv.a;
    if (d.bf16) dg.colsum = ws.part;  // db_fc1's column sums of dA per 128 rows
    const GemmArgs wg = plain(dy, d.h, sv.z, d.ft, dw2, d.ft, d.h, d.ft, d.M);
    return gemm_dgrad_wgrad(d, dg, EPI_DGELU, wg, stream);
  });
  q.run("db_fc1", 0, d.bf16 ? 4.0 * gemm_colsum_floats((int)d.M, (int)d.ft) : (double)d.M * d.ft * d.es, [&] {
    if (d.bf16)
      return launch_colsum_final(ws.part, db1, ((int)d.M + kColsumRows - 1) / kColsumRows, (int)d.ft, stream);
    return launch_colsum(d.bf16, 0, ws.da, false, nullptr, false, nullptr, nullptr, db1, nullptr, ws.part, (int)d.M,
                         (int)d.ft, stream);
  });
  q.run("fc1_dgrad_wgrad", 2 * gflop(d.M, d.h, d.ft), 0, [&] {
    const GemmArgs dg = plain(ws.da, d.ft, w1, d.h, dx, d.h, d.M, d.h, d.ft);
    const GemmArgs wg = plain(ws.da, d.ft, x, d.h, dw1, d.h, d.ft, d.h, d.M);
    return gemm_dgrad_wgrad(d, dg, EPI_STORE, wg, stream);
  });
  return q.status();
}

// ------------------------------------------------------------------------- attention block
// Activation store of mt_attn_fwd -> mt_attn_bwd and the workspace either needs.
size_t carve_attn_saved(const Dims& d, void* base, AttnBufs* b) {
  Carver c(base);
  b->qkv = c.take(d.M * d.qkv * d.es);
  b->p = d.flash ? nullptr : c.take(d.B * d.at * d.seq * d.seq * d.es);
  b->lse = d.flash ? c.take<float>(d.B * d.at * d.seq * 4) : nullptr;
  b->qkv_lo_saved = nullptr;
  b->ctx = c.take(d.M * d.hs * d.es);
  return c.off;
}
size_t carve_attn_fwd_ws(const Dims& d, void* base, AttnBufs* b) {
  Carver c(base);
  b->S = d.flash ? nullptr : c.take<float>(d.B * d.at * d.seq * d.seq * 4);
  b->qkv_lo_ws = nullptr;
  return c.off;
}
size_t carve_attn_bwd_ws(const Dims& d, void* base, AttnBwdWs* w) {
  Carver c(base);
  w->dctx = c.take(d.M * d.hs * d.es);
  w->ds = d.flash ? nullptr : c.take(d.B * d.at * d.seq * d.seq * d.es);
  w->dqkv = c.take(d.M * d.qkv * d.es);
  w->D = c.take<float>(d.B * d.at * d.seq * 4);
  size_t np = colsum_partial_floats((int)d.M, (int)d.qkv, 0);
  if (d.flash) np = std::max(np, (size_t)(flash_dbias_rows((int)d.B, (int)d.seq) * d.qkv));
  w->part = c.take<float>(np * 4);
  const int64_t sp = dgrad_split_floats(d);
  w->spart = sp ? c.take<float>(sp * 4) : nullptr;
  return c.off;
}
size_t attn_ws_bytes(const Dims& d) {
  AttnBufs b;
  AttnBwdWs w;
  return std::max(carve_attn_fwd_ws(d, nullptr, &b), carve_attn_bwd_ws(d, nullptr, &w));
}

// ------------------------------------------------------------------------- sequence-parallel rows
// The rank's share of the tokens under sequence parallelism: seq / tp positions of each
// of the micro_batch sequences (seq must split evenly). The attention block has no
// MT_BF16_QK form (its input arrives already rounded), so neither do these calls.
int validate_sp(const mt_shape* s, Dims* d, int* rows) {
  const int st = validate_shape(s, d);
  if (st != MT_OK) return st;
  if (d->comp) return MT_ERR_UNSUPPORTED;
  if (s->seq % s->tp != 0) return MT_ERR_INVALID_ARG;
  *rows = (int)(d->M / d->tp);
  return MT_OK;
}
size_t sp_ln_ws_floats(int rows, int h) {
  size_t n = std::max(colsum_partial_floats(rows, h, 1), colsum_partial_floats(rows, h, 0));
  if (ln_bwd_sums_supported(h)) n = std::max(n, ln_bwd_sums_partial_floats(rows, h, 4));
  return n;
}
bool null_or_aligned(const void* p) { return !p || aligned16(p); }

bool weights_ok(const mt_layer_weights* w) {
  if (!w) return false;
  const void* p[] = {w->ln1_g, w->ln1_b, w->w_qkv, w->b_qkv, w->w_o,   w->b_o,
                     w->ln2_g, w->ln2_b, w->w_fc1, w->b_fc1, w->w_fc2, w->b_fc2};
  for (const void* q : p)
    if (!aligned16(q)) return false;
  return true;
}

bool grads_ok(const mt_layer_grads* g) {
  if (!g) return false;
  const void* p[] = {g->ln1_g, g->ln1_b, g->w_qkv, g->b_qkv, g->w_o,   g->b_o,
                     g->ln2_g, g->ln2_b, g->w_fc1, g->b_fc1, g->w_fc2, g->b_fc2};
  for (const void* q : p)
    if (!aligned16(q)) return false;
  return true;
}

// ------------------------------------------------------------------------- static scratch
// The workspace of mt_mlp_bwd_noalloc: a fixed device array in the library's code
// object, allocated by the HIP runtime when it loads the module on a device and held
// until the process ends. Host code never uses the array's name as an address (on the
// host it is a stand-in symbol): scratch_address asks the runtime for the current
// device's copy once per device and keeps it.
constexpr size_t kNoallocScratchBytes = (size_t)MT_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch`; the stream (if any) must belong to that
// device. Returns MT_OK, MT_ERR_INVALID_ARG (stream of another device) or MT_ERR_HIP.
int scratch_address(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MT_ERR_HIP;
  if (stream) {
    int sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return MT_ERR_HIP;
    if (sdev != dev) return MT_ERR_INVALID_ARG;
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MT_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MT_OK;
}

}  // namespace
}  // namespace mt

using namespace mt;

extern "C" {

size_t mt_layer_saved_bytes(const mt_shape* shape) {
  Dims d;
  if (validate_shape(shape, &d) != MT_OK) return 0;
  LayerSaved s;
  return carve_layer_saved(d, nullptr, &s);
}

size_t mt_layer_workspace_bytes(const mt_shape* shape) {
  Dims d;
  if (validate_shape(shape, &d) != MT_OK) return 0;
  LayerFwdWs f;
  LayerBwdWs b;
  return std::max(carve_layer_fwd_ws(d, nullptr, &f), carve_layer_bwd_ws(d, nullptr, &b));
}

int mt_layer_fwd(const mt_shape* shape, const mt_layer_weights* w, const void* x, void* out, void* saved,
                 size_t saved_bytes, void* workspace, size_t workspace_bytes, void* stream) {
  Dims d;
  int st = validate_shape(shape, &d);
  if (st != MT_OK) return st;
  if (!weights_ok(w) || !aligned16(x) || !aligned16(out) || !aligned16(saved) || !aligned16(workspace))
    return MT_ERR_INVALID_ARG;
  LayerSaved sv;
  LayerFwdWs ws;
  if (saved_bytes < carve_layer_saved(d, nullptr, &sv) || workspace_bytes < mt_layer_workspace_bytes(shape))
    return MT_ERR_WORKSPACE;
  carve_layer_saved(d, saved, &sv);
  carve_layer_fwd_ws(d, workspace, &ws);
  return layer_fwd_impl(d, *w, x, out, sv, ws, static_cast<hipStream_t>(stream));
}

int mt_layer_bwd(const mt_shape* shape, const mt_layer_weights* w, const void* x, const void* saved,
                 size_t saved_bytes, const void* dout, void* dx, const mt_layer_grads* grads, void* workspace,
                 size_t workspace_bytes, void* stream) {
  Dims d;
  int st = validate_shape(shape, &d);
  if (st != MT_OK) return st;
  if (!weights_ok(w) || !grads_ok(grads) || !aligned16(x) || !aligned16(saved) || !aligned16(dout) ||
      !aligned16(dx) || !aligned16(workspace))
    return MT_ERR_INVALID_ARG;
  LayerSaved sv;
  LayerBwdWs ws;
  if (saved_bytes < carve_layer_saved(d, nullptr, &sv) || workspace_bytes < mt_layer_workspace_bytes(shape))
    return MT_ERR_WORKSPACE;
  carve_layer_saved(d, const_cast<void*>(saved), &sv);
  carve_layer_bwd_ws(d, workspace, &ws);
  return layer_bwd_impl(d, *w, x, sv, dout, dx, *grads, ws, static_cast<hipStream_t>(stream));
}

size_t mt_mlp_saved_bytes(const mt_shape* shape) {
  Dims d;
  if (validate_shape(shape, &d) != MT_OK) return 0;
  MlpSaved s;
  return carve_mlp_saved(d, nullptr, &s);
}

size_t mt_mlp_workspace_bytes(const mt_shape* shape) {
  Dims d;
  if (validate_shape(shape, &d) != MT_OK) return 0;
  MlpWs w;
  return carve_mlp_ws(d, nullptr, &w);
}

int mt_mlp_fwd(const mt_shape* shape, const void* x, const void* w_fc1, const void* b_fc1, const void* w_fc2,
               void* y_partial, void* saved, size_t saved_bytes, void* workspace, size_t workspace_bytes,
               void* stream) {
  Dims d;
  int st = validate_shape(shape, &d);
  if (st != MT_OK) return st;
  (void)workspace;
  if (!aligned16(x) || !aligned16(w_fc1) || !aligned16(b_fc1) || !aligned16(w_fc2) || !aligned16(y_partial) ||
      !aligned16(saved))
    return MT_ERR_INVALID_ARG;
  if (workspace && !aligned16(workspace)) return MT_ERR_INVALID_ARG;
  MlpSaved sv;
  if (saved_bytes < carve_mlp_saved(d, nullptr, &sv)) return MT_ERR_WORKSPACE;
  (void)workspace_bytes;  // the forward needs no scratch
  carve_mlp_saved(d, saved, &sv);
  return mlp_fwd_impl(d, x, w_fc1, b_fc1, w_fc2, y_partial, sv, static_cast<hipStream_t>(stream));
}

int mt_mlp_bwd(const mt_shape* shape, const void* x, const void* w_fc1, const void* w_fc2, const void* saved,
               size_t saved_bytes, const void* dy, void* dx_partial, float* dw_fc1, float* db_fc1, float* dw_fc2,
               void* workspace, size_t workspace_bytes, void* stream) {
  Dims d;
  int st = validate_shape(shape, &d);
  if (st != MT_OK) return st;
  if (!aligned16(x) || !aligned16(w_fc1) || !aligned16(w_fc2) || !aligned16(saved) || !aligned16(dy) ||
      !aligned16(dx_partial) || !aligned16(dw_fc1) || !aligned16(db_fc1) || !aligned16(dw_fc2) ||
      !aligned16(workspace))
    return MT_ERR_INVALID_ARG;
  MlpSaved sv;
  MlpWs ws;
  if (saved_bytes < carve_mlp_saved(d, nullptr, &sv) || workspace_bytes < carve_mlp_ws(d, nullptr, &ws))
    return MT_ERR_WORKSPACE;
  carve_mlp_saved(d, const_cast<void*>(saved), &sv);
  carve_mlp_ws(d, workspace, &ws);
  return mlp_bwd_impl(d, x, w_fc1, w_fc2, sv, dy, dx_partial, dw_fc1, db_fc1, dw_fc2, ws,
                      static_cast<hipStream_t>(stream));
}

int mt_mlp_bwd_noalloc(const mt_shape* shape, const void* x, const void* w_fc1, const void* w_fc2, const void* saved,
                       size_t saved_bytes, const void* dy, void* dx_partial, float* dw_fc1, float* db_fc1,
                       float* dw_fc2, void* stream) {
  Dims d;
  int st = validate_shape(shape, &d);
  if (st != MT_OK) return st;
  if (!aligned16(x) || !aligned16(w_fc1) || !aligned16(w_fc2) || !aligned16(saved) || !aligned16(dy) ||
      !aligned16(dx_partial) || !aligned16(dw_fc1) || !aligned16(db_fc1) || !aligned16(dw_fc2))
    return MT_ERR_INVALID_ARG;
  MlpSaved sv;
  MlpWs ws;
  if (saved_bytes < carve_mlp_saved(d, nullptr, &sv)) return MT_ERR_WORKSPACE;
  if (carve_mlp_ws(d, nullptr, &ws) > kNoallocScratchBytes) return MT_ERR_NOALLOC_LIMIT;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  void* base = nullptr;
  st = scratch_address(s, &base);
  if (st != MT_OK) return st;
  carve_mlp_saved(d, const_cast<void*>(saved), &sv);
  carve_mlp_ws(d, base, &ws);
  return mlp_bwd_impl(d, x, w_fc1, w_fc2, sv, dy, dx_partial, dw_fc1, db_fc1, dw_fc2, ws, s, /*no_timing=*/true);
}

size_t mt_attn_saved_bytes(const mt_shape* shape) {
  Dims d;
  if (validate_shape(shape, &d) != MT_OK || d.comp) return 0;
  AttnBufs b;
  return carve_attn_saved(d, nullptr, &b);
}

size_t mt_attn_workspace_bytes(const mt_shape* shape) {
  Dims d;
  if (validate_shape(shape, &d) != MT_OK || d.comp) return 0;
  return attn_ws_bytes(d);
}

int mt_attn_fwd(const mt_shape* shape, const void* u, const void* w_qkv, const void* b_qkv, const void* w_o,
                void* o_partial, void* saved, size_t saved_bytes, void* workspace, size_t workspace_bytes,
                void* stream) {
  Dims d;
  const int st = validate_shape(shape, &d);
  if (st != MT_OK) return st;
  if (d.comp) return MT_ERR_UNSUPPORTED;
  if (!aligned16(u) || !aligned16(w_qkv) || !aligned16(b_qkv) || !aligned16(w_o) || !aligned16(o_partial) ||
      !aligned16(saved) || !aligned16(workspace))
    return MT_ERR_INVALID_ARG;
  AttnBufs b;
  if (saved_bytes < carve_attn_saved(d, nullptr, &b) || workspace_bytes < attn_ws_bytes(d)) return MT_ERR_WORKSPACE;
  carve_attn_saved(d, saved, &b);
  carve_attn_fwd_ws(d, workspace, &b);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  Seq q(s);
  attn_fwd_part(q, d, u, nullptr, w_qkv, b_qkv, w_o, b, o_partial, s);
  return q.status();
}

int mt_attn_bwd(const mt_shape* shape, const void* u, const void* w_qkv, const void* w_o, const void* saved,
                size_t saved_bytes, const void* d_o, void* du_partial, float* dw_qkv, float* db_qkv, float* dw_o,
                void* workspace, size_t workspace_bytes, void* stream) {
  Dims d;
  const int st = validate_shape(shape, &d);
  if (st != MT_OK) return st;
  if (d.comp) return MT_ERR_UNSUPPORTED;
  if (!aligned16(u) || !aligned16(w_qkv) || !aligned16(w_o) || !aligned16(saved) || !aligned16(d_o) ||
      !aligned16(du_partial) || !aligned16(dw_qkv) || !aligned16(db_qkv) || !aligned16(dw_o) ||
      !aligned16(workspace))
    return MT_ERR_INVALID_ARG;
  AttnBufs b;
  if (saved_bytes < carve_attn_saved(d, nullptr, &b) || workspace_bytes < attn_ws_bytes(d)) return MT_ERR_WORKSPACE;
  carve_attn_saved(d, const_cast<void*>(saved), &b);
  AttnBwdWs w;
  carve_attn_bwd_ws(d, workspace, &w);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  Seq q(s);
  attn_bwd_part(q, d, u, w_qkv, w_o, b, d_o, du_partial, dw_qkv, db_qkv, dw_o, w, s);
  return q.status();
}

int mt_sp_ln_fwd(const mt_shape* shape, const void* x, const void* resid, const void* bias, const void* gamma,
                 const void* beta, float* x2, void* y, float* mean, float* rstd, void* stream) {
  Dims d;
  int rows = 0;
  const int st = validate_sp(shape, &d, &rows);
  if (st != MT_OK) return st;
  if (!aligned16(x) || !aligned16(gamma) || !aligned16(beta) || !aligned16(y) || !aligned16(mean) ||
      !aligned16(rstd) || !null_or_aligned(resid))
    return MT_ERR_INVALID_ARG;
  if (resid && (!aligned16(bias) || !aligned16(x2))) return MT_ERR_INVALID_ARG;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  Seq q(s);
  const double rh = (double)rows * d.h, es = (double)d.es;
  if (!resid) {
    q.run("sp_ln1_fwd", 0, rh * 2 * es, [&] {
      return launch_ln_fwd(d.bf16, x, gamma, beta, y, nullptr, mean, rstd, rows, (int)d.h, kLnEps, s);
    });
  } else {
    q.run("sp_add_ln2_fwd", 0, rh * (3 * es + 4), [&] {
      return launch_add_ln_fwd(d.bf16, x, resid, bias, gamma, beta, x2, y, mean, rstd, rows, (int)d.h, kLnEps, s);
    });
  }
  return q.status();
}

int mt_sp_add_fwd(const mt_shape* shape, const float* x2, const void* y, const void* bias, void* out, void* stream) {
  Dims d;
  int rows = 0;
  const int st = validate_sp(shape, &d, &rows);
  if (st != MT_OK) return st;
  if (!aligned16(x2) || !aligned16(y) || !aligned16(bias) || !aligned16(out)) return MT_ERR_INVALID_ARG;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  Seq q(s);
  q.run("sp_bias_residual_fwd", 0, (double)rows * d.h * (2 * d.es + 4), [&] {
    return launch_add_bias_residual(d.bf16, x2, y, bias, out, rows, (int)d.h, s);
  });
  return q.status();
}

size_t mt_sp_ln_workspace_bytes(const mt_shape* shape) {
  Dims d;
  int rows = 0;
  if (validate_sp(shape, &d, &rows) != MT_OK) return 0;
  return sp_ln_ws_floats(rows, (int)d.h) * 4;
}

int mt_sp_ln_bwd(const mt_shape* shape, const void* dy, const void* xin, int xin_f32, const void* gamma,
                 const float* mean, const float* rstd, const void* dres, int dres_f32, void* dx, float* dx_f32,
                 float* dgamma, float* dbeta, float* dsum, float* dres_sum, void* workspace, size_t workspace_bytes,
                 void* stream) {
  Dims d;
  int rows = 0;
  const int st = validate_sp(shape, &d, &rows);
  if (st != MT_OK) return st;
  if (!aligned16(dy) || !aligned16(xin) || !aligned16(gamma) || !aligned16(mean) || !aligned16(rstd) ||
      !aligned16(dres) || !aligned16(dx) || !aligned16(dgamma) || !aligned16(dbeta) || !aligned16(workspace) ||
      !null_or_aligned(dx_f32) || !null_or_aligned(dsum) || !null_or_aligned(dres_sum))
    return MT_ERR_INVALID_ARG;
  if (dsum && !dx_f32) return MT_ERR_INVALID_ARG;  // the sum of dx is taken over its fp32 values
  if (workspace_bytes < sp_ln_ws_floats(rows, (int)d.h) * 4) return MT_ERR_WORKSPACE;
  float* part = static_cast<float*>(workspace);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int h = (int)d.h;
  const double rh = (double)rows * d.h, es = (double)d.es;
  const double xb = xin_f32 ? 4 : es, rb = dres_f32 ? 4 : es;
  Seq q(s);
  const bool fused = ln_bwd_sums_supported(h);
  if (fused) {  // dres_sum rides along (or follows as a column sum inside the same call)
    q.run("sp_ln_bwd", 0, rh * (es + xb + rb + es + (dx_f32 ? 4 : 0)), [&] {
      return launch_ln_bwd_sums(d.bf16, dy, xin, xin_f32 != 0, gamma, mean, rstd, dres, dres_f32 != 0, dx, dx_f32,
                                part, dgamma, dbeta, dsum, dres_sum, rows, h, s);
    });
  } else {
    q.run("sp_ln_bwd", 0, rh * (es + xb + rb + es + (dx_f32 ? 4 : 0)), [&] {
      return launch_ln_bwd(d.bf16, dy, xin, xin_f32 != 0, gamma, mean, rstd, dres, dres_f32 != 0, dx, dx_f32, rows,
                           h, s);
    });
    q.run("sp_ln_param_grads", 0, rh * (es + xb), [&] {
      return launch_colsum(d.bf16, 1, dy, false, xin, xin_f32 != 0, mean, rstd, dgamma, dbeta, part, rows, h, s);
    });
    if (dsum)
      q.run("sp_ln_dsum", 0, rh * 4, [&] {
        return launch_colsum(d.bf16, 0, dx_f32, true, nullptr, false, nullptr, nullptr, dsum, nullptr, part, rows, h,
                             s);
      });
  }
  if (dres_sum && !fused)
    q.run("sp_dres_sum", 0, rh * rb, [&] {
      return launch_colsum(d.bf16, 0, dres, dres_f32 != 0, nullptr, false, nullptr, nullptr, dres_sum, nullptr, part,
                           rows, h, s);
    });
  return q.status();
}

int mt_adamw_step(int64_t n, float* param, const float* grad, float* exp_avg, float* exp_avg_sq, void* param_bf16,
                  float lr, float beta1, float beta2, float eps, float weight_decay, float grad_scale, int32_t step,
                  void* stream) {
  if (n < 0 || step < 1 || !(beta1 >= 0.f && beta1 < 1.f) || !(beta2 >= 0.f && beta2 < 1.f))
    return MT_ERR_INVALID_ARG;
  if (n == 0) return MT_OK;
  if (!aligned16(param) || !aligned16(grad) || !aligned16(exp_avg) || !aligned16(exp_avg_sq) ||
      (param_bf16 && !aligned16(param_bf16)))
    return MT_ERR_INVALID_ARG;
  AdamwArgs a;
  a.p = param;
  a.g = grad;
  a.m = exp_avg;
  a.v = exp_avg_sq;
  a.p16 = param_bf16;
  a.n = n;
  a.grad_scale = grad_scale;
  a.beta1 = beta1;
  a.one_minus_beta1 = (float)(1.0 - (double)beta1);
  a.beta2 = beta2;
  a.one_minus_beta2 = (float)(1.0 - (double)beta2);
  a.lr_wd = (float)((double)lr * (double)weight_decay);
  // bias corrections of the zero-initialised moments, in double on the host
  a.step_size = (float)((double)lr / (1.0 - std::pow((double)beta1, (double)step)));
  a.inv_sqrt_bc2 = (float)(1.0 / std::sqrt(1.0 - std::pow((double)beta2, (double)step)));
  a.eps = eps;
  const double bytes = (double)n * (28.0 + (param_bf16 ? 2.0 : 0.0));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  Seq q(s);
  q.run("adamw", 0.0, bytes, [&] { return launch_adamw(a, s); });
  return q.status();
}

const char* mt_status_string(int status) {
  switch (status) {
    case MT_OK: return "ok";
    case MT_ERR_INVALID_ARG: return "invalid argument (null or misaligned pointer, or inconsistent shape)";
    case MT_ERR_UNSUPPORTED: return "unsupported shape (head dim or seq not a multiple of 8, seq > 4096, h too large)";
    case MT_ERR_HIP: return "HIP launch or runtime error";
    case MT_ERR_WORKSPACE: return "saved or workspace buffer smaller than the *_bytes query";
    case MT_ERR_NOALLOC_LIMIT:
      return "the shape needs more scratch than the static no-alloc buffer holds (MT_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int mt_timing_enable(int enable, const char* label_filter) {
  std::lock_guard<std::mutex> lk(g_tmu);
  g_filter = label_filter ? label_filter : "";
  g_timing.store(enable != 0, std::memory_order_release);
  return MT_OK;
}

int mt_timing_reset(void) {
  std::lock_guard<std::mutex> lk(g_tmu);
  for (auto& r : g_recs) {
    g_free.push_back(r.a);
    g_free.push_back(r.b);
  }
  g_recs.clear();
  return MT_OK;
}

int mt_timing_count(void) {
  std::lock_guard<std::mutex> lk(g_tmu);
  return (int)g_recs.size();
}

int mt_timing_get(int i, char* label, size_t label_len, float* ms, double* flops, double* bytes) {
  TimingRec r;
  {
    std::lock_guard<std::mutex> lk(g_tmu);
    if (i < 0 || i >= (int)g_recs.size()) return MT_ERR_INVALID_ARG;
    r = g_recs[i];
  }
  if (label && label_len > 0) {
    std::strncpy(label, r.label.c_str(), label_len - 1);
    label[label_len - 1] = '\0';
  }
  if (hipEventSynchronize(r.b) != hipSuccess) return MT_ERR_HIP;
  float t = 0.f;
  if (hipEventElapsedTime(&t, r.a, r.b) != hipSuccess) return MT_ERR_HIP;
  if (ms) *ms = t;
  if (flops) *flops = r.flops;
  if (bytes) *bytes = r.bytes;
  return MT_OK;
}

}  // extern "C"
