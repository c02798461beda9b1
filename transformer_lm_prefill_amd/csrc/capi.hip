// C ABI of the layer library: argument checks, workspace layout, the launch sequence of one
// decoder layer on the caller's stream, error reporting and optional per-kernel timing.
//
// Argument rules follow the pages' own checks where they have them (hf2q 0.1.1,
// qwen3vl_text/forward.rs, `forward_text_prefill_logits_last`: an empty sequence is an error,
// the DeepStack rows must lie inside the sequence, a slab needs rows) and fail loudly on any
// shape the kernels do not run: there is no fallback path.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.h"
#include "qwen3_prefill.h"

namespace {

thread_local std::string g_err;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return status;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(QWEN3_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// ---- per-kernel timing --------------------------------------------------------------------
constexpr int kMaxTimed = 65536;
std::mutex g_tmu;
bool g_timing = false;
std::vector<hipEvent_t> g_events;           // 2 per slot, created on demand and reused
std::vector<const char*> g_slot_name;       // name of the kernel timed in each used slot
int g_used = 0;

int timing_begin(const char* name, hipStream_t s) {
  std::lock_guard<std::mutex> lk(g_tmu);
  if (!g_timing || g_used >= kMaxTimed) return -1;
  const int slot = g_used;
  while (static_cast<int>(g_events.size()) < 2 * (slot + 1)) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return -1;
    g_events.push_back(e);
  }
  if (static_cast<int>(g_slot_name.size()) <= slot) g_slot_name.resize(slot + 1);
  g_slot_name[slot] = name;
  if (hipEventRecord(g_events[2 * slot], s) != hipSuccess) return -1;
  ++g_used;
  return slot;
}

void timing_end(int slot, hipStream_t s) {
  std::lock_guard<std::mutex> lk(g_tmu);
  (void)hipEventRecord(g_events[2 * slot + 1], s);
}

struct KTimer {
  int slot = -1;
  hipStream_t s;
  KTimer(const char* name, hipStream_t st) : s(st) {
    if (g_timing) slot = timing_begin(name, st);
  }
  ~KTimer() {
    if (slot >= 0) timing_end(slot, s);
  }
};

// ---- checks ---------------------------------------------------------------------------------
bool valid_dtype(int d) { return d == QWEN3_F32 || d == QWEN3_BF16 || d == QWEN3_F16; }
// Weight storage formats: the element types, plus fp16 with tiled projection matrices.
bool valid_wdtype(int d) { return valid_dtype(d) || d == QWEN3_F16_TILED; }
// Element type of the weight vectors (norms), embeddings and DeepStack slabs under wdtype w.
qwen3_dtype plain_w(qwen3_dtype w) { return w == QWEN3_F16_TILED ? QWEN3_F16 : w; }
size_t round16(int32_t n) { return (static_cast<size_t>(n) + 15) & ~static_cast<size_t>(15); }
size_t dsize(qwen3_dtype d) { return d == QWEN3_F32 ? 4 : 2; }

// (weights, product operands) pairs the kernels run: f32/f32, bf16/bf16, bf16/f16, f16/f16.
int check_formats(qwen3_dtype w, qwen3_dtype a) {
  if (!valid_wdtype(w) || !valid_dtype(a))
    return fail(QWEN3_ERR_INVALID_ARG, "dtype (%d, %d) is not a qwen3_dtype", w, a);
  const bool ok = (w == QWEN3_F32 && a == QWEN3_F32) || (w == QWEN3_BF16 && a == QWEN3_BF16) ||
                  (w == QWEN3_BF16 && a == QWEN3_F16) || (w == QWEN3_F16 && a == QWEN3_F16) ||
                  (w == QWEN3_F16_TILED && a == QWEN3_F16);
  if (!ok)
    return fail(QWEN3_ERR_UNSUPPORTED,
                "weights %d with operands %d: supported pairs are f32/f32, bf16/bf16, bf16/f16, f16/f16, "
                "f16-tiled/f16", w, a);
  return QWEN3_OK;
}
size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

// Kernels move rows in 16-byte vectors: every tensor pointer must be 16-byte aligned.
bool misaligned16(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (p && reinterpret_cast<uintptr_t>(p) % 16 != 0) return true;
  return false;
}

int check_heads(int32_t nh, int32_t nkv, int32_t hd, qwen3_dtype dt) {
  const char* dname = dt == QWEN3_F16 ? "f16" : "bf16";
  if (nh < 1 || nkv < 1) return fail(QWEN3_ERR_INVALID_ARG, "n_heads (%d) and n_kv_heads (%d) must be >= 1", nh, nkv);
  if (nh % nkv != 0)
    return fail(QWEN3_ERR_INVALID_ARG, "n_heads (%d) must be a multiple of n_kv_heads (%d)", nh, nkv);
  if (dt != QWEN3_F32) {
    const int g = nh / nkv;
    if (hd != 64 && hd != 128) return fail(QWEN3_ERR_UNSUPPORTED, "%s head_dim must be 64 or 128 (got %d)", dname, hd);
    if (g != 1 && g != 2 && g != 4 && g != 8)
      return fail(QWEN3_ERR_UNSUPPORTED, "%s n_heads / n_kv_heads must be 1, 2, 4 or 8 (got %d)", dname, g);
  } else {
    if (hd != 64 && hd != 128) return fail(QWEN3_ERR_UNSUPPORTED, "f32 head_dim must be 64 or 128 (got %d)", hd);
  }
  return QWEN3_OK;
}

int check_sections(const int32_t sec[3], int32_t hd) {
  if (!sec) return fail(QWEN3_ERR_INVALID_ARG, "mrope_section is NULL");
  const int half = hd / 2;
  if (sec[0] < 0 || sec[1] < 0 || sec[2] < 0 || sec[0] + sec[1] + sec[2] != half)
    return fail(QWEN3_ERR_INVALID_ARG, "mrope_section (%d,%d,%d) must be >= 0 and sum to head_dim/2 = %d",
                sec[0], sec[1], sec[2], half);
  if (3 * sec[1] > half || 3 * sec[2] > half)
    return fail(QWEN3_ERR_INVALID_ARG,
                "mrope_section h (%d) and w (%d) must be <= head_dim/6 for the interleaved layout", sec[1], sec[2]);
  return QWEN3_OK;
}

// DeepStack rows: a HOST array of n_ds strictly increasing row indices in [0, S) (hf2q
// forward.rs, `forward_text_prefill_logits_last`: an image-token position outside the sequence
// is an error; a slab needs its rows).
int check_ds_rows(const int32_t* rows, int32_t n_ds, int32_t S) {
  if (n_ds < 0 || n_ds > S) return fail(QWEN3_ERR_INVALID_ARG, "n_ds (%d) must be in [0, seq_len = %d]", n_ds, S);
  if (n_ds > 0 && !rows) return fail(QWEN3_ERR_INVALID_ARG, "n_ds = %d needs the host row list ds_rows", n_ds);
  for (int32_t i = 0; i < n_ds; ++i) {
    if (rows[i] < 0 || rows[i] >= S)
      return fail(QWEN3_ERR_INVALID_ARG, "DeepStack row %d (entry %d) is outside [0, seq_len = %d)", rows[i], i, S);
    if (i > 0 && rows[i] <= rows[i - 1])
      return fail(QWEN3_ERR_INVALID_ARG, "DeepStack rows must be strictly increasing (entry %d: %d after %d)", i,
                  rows[i], rows[i - 1]);
  }
  return QWEN3_OK;
}

int check_cfg(const qwen3_layer_cfg* c) {
  if (!c) return fail(QWEN3_ERR_INVALID_ARG, "cfg is NULL");
  int st = check_formats(c->wdtype, c->act_dtype);
  if (st) return st;
  if (c->resid_dtype != QWEN3_F32)
    return fail(QWEN3_ERR_UNSUPPORTED, "resid_dtype must be QWEN3_F32 (the residual stream is carried in fp32)");
  if (c->hidden < 256 || c->hidden % 256 != 0 || c->hidden > 16384)
    return fail(QWEN3_ERR_UNSUPPORTED, "hidden (%d) must be a multiple of 256 in [256, 16384]", c->hidden);
  if (c->ffn < 128 || c->ffn % 128 != 0)
    return fail(QWEN3_ERR_UNSUPPORTED, "ffn (%d) must be a positive multiple of 128", c->ffn);
  st = check_heads(c->n_heads, c->n_kv_heads, c->head_dim, c->act_dtype);
  if (st) return st;
  if (static_cast<int64_t>(c->n_heads) * c->head_dim > 65536)
    return fail(QWEN3_ERR_UNSUPPORTED, "n_heads * head_dim too large");
  st = check_sections(c->mrope_section, c->head_dim);
  if (st) return st;
  if (!(c->rms_eps >= 0.f) || !std::isfinite(c->rms_eps))
    return fail(QWEN3_ERR_INVALID_ARG, "rms_eps must be finite and >= 0");
  if (!(c->rope_theta > 1.f) || !std::isfinite(c->rope_theta))
    return fail(QWEN3_ERR_INVALID_ARG, "rope_theta must be finite and > 1");
  return QWEN3_OK;
}

struct Workspace {
  size_t xn, qkv, o, act, dsrows, total;
};

// xn, o and act are the A operands of the products: in the tiled layout for 16-bit operands,
// over whole 16-row groups (S rounded up to a multiple of 16).
Workspace layout(const qwen3_layer_cfg* c, int32_t S) {
  const size_t e = dsize(c->act_dtype);
  const size_t q_dim = static_cast<size_t>(c->n_heads) * c->head_dim;
  const size_t kv_dim = static_cast<size_t>(c->n_kv_heads) * c->head_dim;
  const size_t S16 = round16(S);
  Workspace w;
  w.xn = 0;
  w.qkv = w.xn + align256(S16 * c->hidden * e);
  w.o = w.qkv + align256(static_cast<size_t>(S) * (q_dim + 2 * kv_dim) * e);
  w.act = w.o + align256(S16 * q_dim * e);
  w.dsrows = w.act + align256(S16 * c->ffn * e);
  w.total = w.dsrows + align256(static_cast<size_t>(S) * 4);
  return w;
}

// ---- building blocks shared by the layer and the sub-op entry points ------------------------
int run_rmsnorm(const float* x, const void* w, qwen3_dtype wd, void* y, qwen3_dtype yd, int rows,
                int hidden, float eps, hipStream_t s, bool y_tiled = false) {
  KTimer t("rmsnorm", s);
  hipError_t e = q3::launch_rmsnorm(x, w, wd, y, yd, rows, hidden, eps, s, y_tiled);
  return e == hipSuccess ? QWEN3_OK : hip_fail(e, "rmsnorm launch");
}

int run_qk_norm_mrope(const q3::RopeParams& p, int hd, qwen3_dtype dt, hipStream_t s) {
  KTimer t("qk_norm_mrope", s);
  hipError_t e = q3::launch_qk_norm_mrope(p, hd, dt, s);
  return e == hipSuccess ? QWEN3_OK : hip_fail(e, "qk_norm_mrope launch");
}

int run_attention(const void* q, const void* k, const void* v, void* o, int64_t qs, int64_t ks,
                  int64_t vs, int64_t os, int S, int nh, int nkv, int hd, float scale, qwen3_dtype dt,
                  int causal, hipStream_t s, bool o_tiled = false) {
  KTimer t(causal ? "attention" : "attention_bidirectional", s);
  hipError_t e;
  if (dt != QWEN3_F32) {
    q3::AttnParams p{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), qs, ks, vs, os,
                     S, nh, nkv, scale * 1.4426950408889634f, hd, causal, o_tiled ? 1 : 0};
    e = q3::launch_attention_mfma(p, dt == QWEN3_F16 ? q3::OPH_F16 : q3::OPH_BF16, s);
  } else {
    q3::AttnF32Params p{static_cast<const float*>(q), static_cast<const float*>(k),
                        static_cast<const float*>(v), static_cast<float*>(o), qs, ks, vs, os,
                        S, nh, nkv, scale, causal};
    e = q3::launch_attention_f32(p, hd, s);
  }
  return e == hipSuccess ? QWEN3_OK : hip_fail(e, "attention launch");
}

// One projection. For bf16: epi selects the store; for f32 the same meanings on the f32 kernel.
struct Proj {
  const void* A; int64_t lda;
  const void* B0; const void* B1; const void* B2; int nseg0, nseg1; int64_t ldb;
  void* C; int64_t ldc;
  const float* R; int64_t ldr;
  int M, N, K;
  int a_t = 0, b_t = 0, c_t = 0;   // A, B, the SwiGLU output in the tiled layout (16-bit only)
  float act_scale = 1.f, out_scale = 1.f;  // 16-bit products only (GemmParams)
};

// With fp16 operands the SwiGLU activation is stored as 2^-4 * a, and the down product that
// reads it multiplies its sum by 2^4. Both scalings are exact (powers of two, fp16 normal
// range), so the result is unchanged, while activations up to 65504 * 16 (about 1.05e6) stay
// finite instead of overflowing at 65504. bf16 operands carry fp32's exponent range unscaled.
constexpr float kActScaleF16 = 0.0625f;
inline float act_scale_for(qwen3_dtype ad) { return ad == QWEN3_F16 ? kActScaleF16 : 1.f; }

// wd: weight dtype; ad: operand dtype (A, MFMA, 16-bit outputs); q4: the B matrices are Q4_0
// blocks decoded inside the product.
int run_gemm(const char* name, const Proj& g, int epi, qwen3_dtype wd, qwen3_dtype ad, hipStream_t s,
             bool q4 = false) {
  KTimer t(name, s);
  hipError_t e;
  if (ad != QWEN3_F32) {
    q3::GemmParams p{static_cast<const uint16_t*>(g.A), g.lda, static_cast<const uint16_t*>(g.B0),
                     static_cast<const uint16_t*>(g.B1), static_cast<const uint16_t*>(g.B2),
                     g.nseg0, g.nseg1, g.ldb, g.C, g.ldc, g.R, g.ldr, g.M, g.N, g.K, g.a_t, g.b_t, g.c_t,
                     g.act_scale, g.out_scale};
    if (q4)
      e = q3::launch_gemm_mfma_q4(p, epi, ad == QWEN3_F16 ? q3::OPH_F16 : q3::OPH_BF16, 0, s);
    else
      e = q3::launch_gemm_mfma(p, epi, ad == QWEN3_F16 ? q3::OPH_F16 : q3::OPH_BF16, wd == QWEN3_BF16, 0, s);
  } else {
    // f32 SwiGLU: N counts F outputs (the dual kernel multiplies gate and up together)
    q3::GemmF32Params p{static_cast<const float*>(g.A), g.lda, static_cast<const float*>(g.B0),
                        static_cast<const float*>(g.B1), static_cast<const float*>(g.B2),
                        g.nseg0, g.nseg1, g.ldb, static_cast<float*>(g.C), g.ldc, g.R, g.ldr,
                        g.M, epi == q3::EPI_SWIGLU_16 ? g.N / 2 : g.N, g.K};
    e = q3::launch_gemm_f32(p, epi == q3::EPI_SWIGLU_16, s);
  }
  if (e != hipSuccess) return hip_fail(e, name);
  return QWEN3_OK;
}

// a = silu(x Wg^T) * (x Wu^T) into act [S, F]; then out = [R +] a Wd^T.
// wdt may be QWEN3_F16_TILED (tiled weight matrices); x, act and out are row-major.
int run_ffn(const void* x, const void* wg, const void* wu, const void* wd, const float* R, void* out,
            qwen3_dtype out_dt, void* act, int S, int H, int F, qwen3_dtype wdt, qwen3_dtype adt,
            hipStream_t s) {
  const int wt = wdt == QWEN3_F16_TILED;
  wdt = plain_w(wdt);
  Proj gu{x, H, wg, wu, nullptr, 0, 0, H, act, F, nullptr, 0, S, 2 * F, H, 0, wt, 0, act_scale_for(adt)};
  int st = run_gemm("gemm_gate_up_swiglu", gu, q3::EPI_SWIGLU_16, wdt, adt, s);
  if (st) return st;
  Proj dn{act, F, wd, nullptr, nullptr, H, H, F, out, H, R, H, S, H, F, 0, wt, 0, 1.f, 1.f / act_scale_for(adt)};
  const int epi = out_dt == QWEN3_F32 ? q3::EPI_STORE_F32 : q3::EPI_STORE_16;
  return run_gemm(R ? "gemm_down_resid" : "gemm_down", dn, epi, wdt, adt, s);
}

// ---- weights of one layer, dense or quantized ------------------------------------------------
struct MatW {
  int fmt;            // qwen3_wformat
  const void* data;   // dense: cfg.wdtype matrix; Q4_0 blocks; int8 codes
  const float* rs;    // q8 rows: row scales
};
struct LayerW {
  const void *attn_norm, *q_norm, *k_norm, *ffn_norm;
  MatW wq, wk, wv, wo, wg, wu, wd;
};

LayerW dense_layer(const qwen3_layer_weights* w) {
  auto m = [](const void* d) { return MatW{QWEN3_W_DENSE, d, nullptr}; };
  return LayerW{w->attn_norm, w->q_norm, w->k_norm, w->ffn_norm, m(w->wq), m(w->wk), m(w->wv), m(w->wo),
                m(w->w_gate), m(w->w_up), m(w->w_down)};
}

LayerW quant_layer(const qwen3_layer_qweights* w) {
  auto m = [](const qwen3_qmatrix& q) { return MatW{q.format, q.data, q.row_scale}; };
  return LayerW{w->attn_norm, w->q_norm, w->k_norm, w->ffn_norm, m(w->wq), m(w->wk), m(w->wv), m(w->wo),
                m(w->w_gate), m(w->w_up), m(w->w_down)};
}

int check_matrix(const MatW& m, const char* name) {
  if (m.fmt != QWEN3_W_DENSE && m.fmt != QWEN3_W_Q4_0 && m.fmt != QWEN3_W_Q8_ROW)
    return fail(QWEN3_ERR_INVALID_ARG, "weight %s: format %d is not a qwen3_wformat", name, m.fmt);
  if (!m.data) return fail(QWEN3_ERR_INVALID_ARG, "weight %s is NULL", name);
  const uintptr_t a = reinterpret_cast<uintptr_t>(m.data);
  if (m.fmt == QWEN3_W_Q4_0) {
    if (a % 4 != 0) return fail(QWEN3_ERR_INVALID_ARG, "weight %s: Q4_0 blocks must be 4-byte aligned", name);
  } else if (a % 16 != 0) {
    return fail(QWEN3_ERR_INVALID_ARG, "weight %s: tensor pointers must be 16-byte aligned", name);
  }
  if (m.fmt == QWEN3_W_Q8_ROW && (!m.rs || reinterpret_cast<uintptr_t>(m.rs) % 4 != 0))
    return fail(QWEN3_ERR_INVALID_ARG, "weight %s: q8 rows need a 4-byte aligned row_scale", name);
  return QWEN3_OK;
}

// Null and alignment checks of every weight; `quant` tells whether quantized formats are
// allowed (they need 16-bit operands).
int check_layer_w(const LayerW& w, const qwen3_layer_cfg* cfg, bool* any_quant) {
  const void* norms[] = {w.attn_norm, w.q_norm, w.k_norm, w.ffn_norm};
  const char* nn[] = {"attn_norm", "q_norm", "k_norm", "ffn_norm"};
  for (int i = 0; i < 4; ++i) {
    if (!norms[i]) return fail(QWEN3_ERR_INVALID_ARG, "weight %s is NULL", nn[i]);
    if (misaligned16({norms[i]})) return fail(QWEN3_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  }
  const MatW* ms[] = {&w.wq, &w.wk, &w.wv, &w.wo, &w.wg, &w.wu, &w.wd};
  const char* mn[] = {"wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"};
  *any_quant = false;
  for (int i = 0; i < 7; ++i) {
    int st = check_matrix(*ms[i], mn[i]);
    if (st) return st;
    *any_quant = *any_quant || ms[i]->fmt != QWEN3_W_DENSE;
  }
  if (*any_quant && cfg->act_dtype == QWEN3_F32)
    return fail(QWEN3_ERR_UNSUPPORTED, "quantized weights need 16-bit operands (act_dtype f16 or bf16)");
  auto same_class = [](const MatW& a, const MatW& b) { return (a.fmt == QWEN3_W_DENSE) == (b.fmt == QWEN3_W_DENSE); };
  if (!same_class(w.wq, w.wk) || !same_class(w.wq, w.wv))
    return fail(QWEN3_ERR_UNSUPPORTED, "wq, wk and wv must be all dense or all quantized");
  if (w.wg.fmt != w.wu.fmt) return fail(QWEN3_ERR_UNSUPPORTED, "w_gate and w_up must share one format");
  return QWEN3_OK;
}

// Bytes of the buffer the prefill expands quantized matrices into: the largest product group.
size_t dequant_bytes(const qwen3_layer_cfg* c) {
  const size_t e = 2, H = c->hidden, F = c->ffn;
  const size_t q_dim = static_cast<size_t>(c->n_heads) * c->head_dim;
  const size_t kv_dim = static_cast<size_t>(c->n_kv_heads) * c->head_dim;
  size_t m = (q_dim + 2 * kv_dim) * H;
  m = std::max(m, H * q_dim);
  m = std::max(m, 2 * F * H);
  m = std::max(m, H * F);
  return align256(m * e);
}

// The matrices of one product group in one storage type: all dense -> as given (wdt; tiled
// matrices set *b_tiled); all
// Q4_0, with the product's A operand (a_elems 16-bit elements) within the 32-bit offsets of the
// GEMM's buffer loads -> the blocks as given, decoded inside the GEMM (*q4 set); otherwise
// quantized -> expanded back to back into dq in the operand type.
int group_weights(const MatW* const* m, int n, const int* rows, int cols, qwen3_dtype wdt, qwen3_dtype act,
                  char* dq, const void** out, qwen3_dtype* bdt, bool* q4, int64_t a_elems, hipStream_t s,
                  int* b_tiled) {
  *q4 = false;
  *b_tiled = 0;
  if (m[0]->fmt == QWEN3_W_DENSE) {
    for (int i = 0; i < n; ++i) out[i] = m[i]->data;
    *bdt = plain_w(wdt);
    *b_tiled = wdt == QWEN3_F16_TILED;
    return QWEN3_OK;
  }
  bool all_q4 = 2 * a_elems <= 0x7fffffff;
  for (int i = 0; i < n; ++i) all_q4 = all_q4 && m[i]->fmt == QWEN3_W_Q4_0;
  if (all_q4) {
    for (int i = 0; i < n; ++i) out[i] = m[i]->data;
    *bdt = act;
    *q4 = true;
    return QWEN3_OK;
  }
  KTimer t("dequant", s);
  size_t off = 0;
  for (int i = 0; i < n; ++i) {
    const hipError_t e = q3::launch_dequant(m[i]->fmt, m[i]->data, m[i]->rs, rows[i], cols, act, dq + off, s);
    if (e != hipSuccess) return hip_fail(e, "dequant launch");
    out[i] = dq + off;
    off += static_cast<size_t>(rows[i]) * cols * 2;
  }
  *bdt = act;
  return QWEN3_OK;
}

}  // namespace

namespace q3 {
// Sets the thread's error text (for entry points defined in other sources); returns status.
int set_error(int status, const char* msg) { return fail(status, "%s", msg); }
}  // namespace q3

extern "C" {

const char* qwen3_last_error(void) { return g_err.c_str(); }

size_t qwen3_layer_workspace_bytes(const qwen3_layer_cfg* cfg, int32_t seq_len) {
  if (!cfg || seq_len < 1 || !valid_dtype(cfg->act_dtype)) return 0;
  return layout(cfg, seq_len).total;
}

size_t swiglu_ffn_workspace_bytes(int32_t seq_len, int32_t ffn, qwen3_dtype x_dtype) {
  if (seq_len < 1 || ffn < 1 || !valid_dtype(x_dtype)) return 0;
  return align256(static_cast<size_t>(seq_len) * ffn * dsize(x_dtype));
}

// The layer prefill; with k_cache set it also writes k' and v of every position into rows
// 0..seq_len-1 of the caches (capacity rows per KV head). Quantized matrices are expanded into
// a buffer after the layer workspace just before their product.
static int layer_prefill_impl(const qwen3_layer_cfg* cfg, const LayerW& w, const void* x_in,
                              void* x_out, int32_t seq_len, const int32_t* positions,
                              const int32_t* ds_rows, int32_t n_ds, const void* ds, void* k_cache,
                              void* v_cache, int32_t capacity, void* workspace, size_t workspace_bytes,
                              void* stream) {
  int st = check_cfg(cfg);
  if (st) return st;
  if (seq_len < 1) return fail(QWEN3_ERR_INVALID_ARG, "seq_len must be >= 1 (got %d): empty prompt", seq_len);
  bool quant = false;
  if ((st = check_layer_w(w, cfg, &quant))) return st;
  if (!x_in || !x_out) return fail(QWEN3_ERR_INVALID_ARG, "x_in / x_out is NULL");
  if (!positions) return fail(QWEN3_ERR_INVALID_ARG, "positions is NULL");
  if (misaligned16({x_in, x_out, ds}))
    return fail(QWEN3_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  if ((st = check_ds_rows(ds_rows, n_ds, seq_len))) return st;
  if (n_ds == 0 && ds) return fail(QWEN3_ERR_INVALID_ARG, "a DeepStack slab was given with n_ds == 0");
  if (n_ds > 0 && !ds) return fail(QWEN3_ERR_INVALID_ARG, "n_ds = %d needs the slab ds", n_ds);
  const Workspace L = layout(cfg, seq_len);
  const size_t need = L.total + (quant ? dequant_bytes(cfg) : 0);
  if (!workspace || workspace_bytes < need)
    return fail(QWEN3_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu%s)", need, workspace_bytes,
                workspace ? "" : ", NULL pointer");
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(QWEN3_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  {
    const size_t xb = static_cast<size_t>(seq_len) * cfg->hidden * 4;
    const char* a = static_cast<const char*>(x_in);
    const char* b = static_cast<const char*>(x_out);
    if (a != b && a < b + xb && b < a + xb)
      return fail(QWEN3_ERR_INVALID_ARG, "x_out partially overlaps x_in (only x_out == x_in is allowed)");
  }

  hipStream_t s = static_cast<hipStream_t>(stream);
  const qwen3_dtype wdt = plain_w(cfg->wdtype), dt = cfg->act_dtype;
  const int S = seq_len, H = cfg->hidden, nh = cfg->n_heads, nkv = cfg->n_kv_heads, hd = cfg->head_dim;
  const int F = cfg->ffn;
  const int q_dim = nh * hd, kv_dim = nkv * hd, qkv_dim = q_dim + 2 * kv_dim;
  // 16-bit operands: xn / yn, o and act go through the workspace in the tiled layout
  const int at = dt != QWEN3_F32;
  const int64_t S16 = static_cast<int64_t>(round16(S));
  int bt = 0;
  const size_t e = dsize(dt);
  char* ws = static_cast<char*>(workspace);
  void* xn = ws + L.xn;
  char* qkv = ws + L.qkv;
  void* o = ws + L.o;
  void* act = ws + L.act;
  char* dq = ws + L.total;   // expanded quantized matrices (quantized layers only)
  const float* x = static_cast<const float*>(x_in);
  float* y = static_cast<float*>(x_out);
  const void* B[3];
  qwen3_dtype bdt;
  bool q4 = false;

  // a1: input RMSNorm
  if ((st = run_rmsnorm(x, w.attn_norm, wdt, xn, dt, S, H, cfg->rms_eps, s, at))) return st;
  // a2: q | k | v = xn [Wq; Wk; Wv]^T in one product, token-major [S, q_dim + 2 kv_dim]
  {
    const MatW* g[3] = {&w.wq, &w.wk, &w.wv};
    const int rows[3] = {q_dim, kv_dim, kv_dim};
    if ((st = group_weights(g, 3, rows, H, cfg->wdtype, dt, dq, B, &bdt, &q4, S16 * H, s, &bt))) return st;
    Proj p{xn, H, B[0], B[1], B[2], q_dim, q_dim + kv_dim, H, qkv, qkv_dim, nullptr, 0, S, qkv_dim, H, at, bt, 0};
    if ((st = run_gemm("gemm_qkv", p, dt == QWEN3_F32 ? q3::EPI_STORE_F32 : q3::EPI_STORE_16, bdt, dt, s, q4)))
      return st;
  }
  // a3+a4: per-head RMSNorm and interleaved MRoPE on q and k, in place; with caches, the same
  // launch appends k' and v of every position (rows 0..S-1)
  {
    q3::RopeParams p{qkv, qkv + static_cast<size_t>(q_dim) * e, qkv_dim, qkv_dim, S, nh, nkv,
                     w.q_norm, w.k_norm, wdt, positions, cfg->rms_eps,
                     std::log2(static_cast<double>(cfg->rope_theta)), cfg->mrope_section[1],
                     cfg->mrope_section[2]};
    if (k_cache) {
      p.kc = k_cache;
      p.vc = v_cache;
      p.v = qkv + static_cast<size_t>(q_dim + kv_dim) * e;
      p.v_stride = qkv_dim;
      p.capacity = capacity;
      p.row0 = 0;
      p.cache_dt = dt;
    }
    if ((st = run_qk_norm_mrope(p, hd, dt, s))) return st;
  }
  // a5: causal GQA attention -> o [S, q_dim]
  if ((st = run_attention(qkv, qkv + static_cast<size_t>(q_dim) * e, qkv + static_cast<size_t>(q_dim + kv_dim) * e,
                          o, qkv_dim, qkv_dim, qkv_dim, q_dim, S, nh, nkv, hd,
                          1.0f / std::sqrt(static_cast<float>(hd)), dt, 1, s, at)))
    return st;
  // a6: y1 = x + o Wo^T (fp32, into x_out)
  {
    const MatW* g[1] = {&w.wo};
    const int rows[1] = {H};
    if ((st = group_weights(g, 1, rows, q_dim, cfg->wdtype, dt, dq, B, &bdt, &q4, S16 * q_dim, s, &bt))) return st;
    Proj p{o, q_dim, B[0], nullptr, nullptr, H, H, q_dim, y, H, x, H, S, H, q_dim, at, bt, 0};
    if ((st = run_gemm("gemm_o_resid", p, q3::EPI_STORE_F32, bdt, dt, s, q4))) return st;
  }
  // a7: yn = RMSNorm(y1, ffn_norm) (reuses the xn buffer)
  if ((st = run_rmsnorm(y, w.ffn_norm, wdt, xn, dt, S, H, cfg->rms_eps, s, at))) return st;
  // a8: a = silu(yn Wg^T) * (yn Wu^T)
  {
    const MatW* g[2] = {&w.wg, &w.wu};
    const int rows[2] = {F, F};
    if ((st = group_weights(g, 2, rows, H, cfg->wdtype, dt, dq, B, &bdt, &q4, S16 * H, s, &bt))) return st;
    Proj gu{xn, H, B[0], B[1], nullptr, 0, 0, H, act, F, nullptr, 0, S, 2 * F, H, at, bt, at, act_scale_for(dt)};
    if ((st = run_gemm("gemm_gate_up_swiglu", gu, q3::EPI_SWIGLU_16, bdt, dt, s, q4))) return st;
  }
  // a9: y2 = y1 + a Wd^T
  {
    const MatW* g[1] = {&w.wd};
    const int rows[1] = {H};
    if ((st = group_weights(g, 1, rows, F, cfg->wdtype, dt, dq, B, &bdt, &q4, S16 * F, s, &bt))) return st;
    Proj dn{act, F, B[0], nullptr, nullptr, H, H, F, y, H, y, H, S, H, F, at, bt, 0, 1.f, 1.f / act_scale_for(dt)};
    if ((st = run_gemm("gemm_down_resid", dn, q3::EPI_STORE_F32, bdt, dt, s, q4))) return st;
  }
  // a10: DeepStack rows (the validated host row list goes to the workspace on the stream)
  if (n_ds > 0) {
    int32_t* drows = reinterpret_cast<int32_t*>(ws + L.dsrows);
    hipError_t he = hipMemcpyAsync(drows, ds_rows, static_cast<size_t>(n_ds) * 4, hipMemcpyHostToDevice, s);
    if (he != hipSuccess) return hip_fail(he, "DeepStack row upload");
    KTimer t("deepstack_add", s);
    he = q3::launch_deepstack_add(y, drows, ds, wdt, n_ds, S, H, s);
    if (he != hipSuccess) return hip_fail(he, "deepstack_add launch");
  }
  return QWEN3_OK;
}

int qwen3_layer_prefill(const qwen3_layer_cfg* cfg, const qwen3_layer_weights* w, const void* x_in,
                        void* x_out, int32_t seq_len, const int32_t* positions,
                        const int32_t* ds_rows, int32_t n_ds, const void* ds, void* workspace,
                        size_t workspace_bytes, void* stream) {
  if (!w) return fail(QWEN3_ERR_INVALID_ARG, "weights is NULL");
  return layer_prefill_impl(cfg, dense_layer(w), x_in, x_out, seq_len, positions, ds_rows, n_ds, ds, nullptr,
                            nullptr, 0, workspace, workspace_bytes, stream);
}

int qwen3_layer_prefill_kv(const qwen3_layer_cfg* cfg, const qwen3_layer_weights* w, const void* x_in,
                           void* x_out, int32_t seq_len, const int32_t* positions,
                           const int32_t* ds_rows, int32_t n_ds, const void* ds, void* k_cache,
                           void* v_cache, int32_t capacity, void* workspace, size_t workspace_bytes,
                           void* stream) {
  if (!k_cache || !v_cache) return fail(QWEN3_ERR_INVALID_ARG, "k_cache / v_cache is NULL");
  if (k_cache == v_cache) return fail(QWEN3_ERR_INVALID_ARG, "k_cache and v_cache must be different buffers");
  if (misaligned16({k_cache, v_cache})) return fail(QWEN3_ERR_INVALID_ARG, "cache pointers must be 16-byte aligned");
  if (capacity < seq_len)
    return fail(QWEN3_ERR_INVALID_ARG, "capacity (%d) must be >= seq_len (%d)", capacity, seq_len);
  if (!w) return fail(QWEN3_ERR_INVALID_ARG, "weights is NULL");
  return layer_prefill_impl(cfg, dense_layer(w), x_in, x_out, seq_len, positions, ds_rows, n_ds, ds, k_cache,
                            v_cache, capacity, workspace, workspace_bytes, stream);
}

size_t qwen3_layer_quant_workspace_bytes(const qwen3_layer_cfg* cfg, int32_t seq_len) {
  if (!cfg || seq_len < 1 || !valid_dtype(cfg->act_dtype) || cfg->hidden < 1 || cfg->ffn < 1) return 0;
  return layout(cfg, seq_len).total + dequant_bytes(cfg);
}

int qwen3_layer_prefill_quant(const qwen3_layer_cfg* cfg, const qwen3_layer_qweights* w, const void* x_in,
                              void* x_out, int32_t seq_len, const int32_t* positions, const int32_t* ds_rows,
                              int32_t n_ds, const void* ds, void* k_cache, void* v_cache, int32_t capacity,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (!w) return fail(QWEN3_ERR_INVALID_ARG, "weights is NULL");
  if ((k_cache == nullptr) != (v_cache == nullptr))
    return fail(QWEN3_ERR_INVALID_ARG, "k_cache and v_cache must be given together");
  if (k_cache) {
    if (k_cache == v_cache) return fail(QWEN3_ERR_INVALID_ARG, "k_cache and v_cache must be different buffers");
    if (misaligned16({k_cache, v_cache}))
      return fail(QWEN3_ERR_INVALID_ARG, "cache pointers must be 16-byte aligned");
    if (capacity < seq_len)
      return fail(QWEN3_ERR_INVALID_ARG, "capacity (%d) must be >= seq_len (%d)", capacity, seq_len);
  }
  return layer_prefill_impl(cfg, quant_layer(w), x_in, x_out, seq_len, positions, ds_rows, n_ds, ds, k_cache,
                            v_cache, capacity, workspace, workspace_bytes, stream);
}

int dequantize_matrix(const qwen3_qmatrix* m, int32_t rows, int32_t cols, qwen3_dtype out_dtype, void* out,
                      void* stream) {
  if (!m) return fail(QWEN3_ERR_INVALID_ARG, "matrix is NULL");
  const MatW mw{m->format, m->data, m->row_scale};
  int st = check_matrix(mw, "matrix");
  if (st) return st;
  if (mw.fmt == QWEN3_W_DENSE) return fail(QWEN3_ERR_INVALID_ARG, "a dense matrix has nothing to dequantize");
  if (out_dtype != QWEN3_F16 && out_dtype != QWEN3_BF16)
    return fail(QWEN3_ERR_UNSUPPORTED, "out_dtype must be f16 or bf16");
  if (rows < 1 || cols < 1) return fail(QWEN3_ERR_INVALID_ARG, "rows (%d) and cols (%d) must be >= 1", rows, cols);
  if (cols % 64 != 0) return fail(QWEN3_ERR_UNSUPPORTED, "cols (%d) must be a multiple of 64", cols);
  if (!out) return fail(QWEN3_ERR_INVALID_ARG, "out is NULL");
  if (misaligned16({out})) return fail(QWEN3_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  KTimer t("dequant", s);
  const hipError_t e = q3::launch_dequant(mw.fmt, mw.data, mw.rs, rows, cols, out_dtype, out, s);
  return e == hipSuccess ? QWEN3_OK : hip_fail(e, "dequant launch");
}

// ---- whole-model prefill to the last position's logits --------------------------------------
struct ModelWorkspace {
  size_t tokens, x, xlast, layer, total;
};

static ModelWorkspace model_layout(const qwen3_model_cfg* c, int32_t S) {
  ModelWorkspace m{};
  const int H = c->layer.hidden;
  m.tokens = 0;
  m.x = align256(static_cast<size_t>(S) * 4);
  m.xlast = m.x + align256(static_cast<size_t>(S) * H * 4);
  m.layer = m.xlast + align256(static_cast<size_t>(H) * 4);
  m.total = m.layer + qwen3_layer_workspace_bytes(&c->layer, S);
  return m;
}

size_t qwen3_model_workspace_bytes(const qwen3_model_cfg* cfg, int32_t seq_len) {
  if (!cfg || seq_len < 1 || qwen3_layer_workspace_bytes(&cfg->layer, seq_len) == 0) return 0;
  return model_layout(cfg, seq_len).total;
}

static int check_model(const qwen3_model_cfg* cfg, const qwen3_model_weights* w, const float* logits) {
  if (!cfg) return fail(QWEN3_ERR_INVALID_ARG, "cfg is NULL");
  int st = check_cfg(&cfg->layer);
  if (st) return st;
  if (cfg->n_layers < 0) return fail(QWEN3_ERR_INVALID_ARG, "n_layers (%d) must be >= 0", cfg->n_layers);
  if (cfg->vocab < 1) return fail(QWEN3_ERR_INVALID_ARG, "vocab (%d) must be >= 1", cfg->vocab);
  if (!w || !w->token_embd || !w->output_norm || (cfg->n_layers > 0 && !w->layers))
    return fail(QWEN3_ERR_INVALID_ARG, "model weights (token_embd, output_norm, layers) must not be NULL");
  if (!logits) return fail(QWEN3_ERR_INVALID_ARG, "logits is NULL");
  if (misaligned16({w->token_embd, w->output_norm, w->lm_head, logits}))
    return fail(QWEN3_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  return QWEN3_OK;
}

// Per-layer caches of a model call: host arrays of n_layers device pointers, both given or both
// NULL; each layer's two caches distinct and 16-byte aligned.
static int check_model_caches(const qwen3_model_cfg* cfg, void* const* kc, void* const* vc, int32_t capacity,
                              int32_t need_rows, bool required) {
  if (cfg->n_layers == 0) return QWEN3_OK;  // no layer, no cache
  if ((kc == nullptr) != (vc == nullptr)) return fail(QWEN3_ERR_INVALID_ARG, "k_caches and v_caches go together");
  if (!kc) return required ? fail(QWEN3_ERR_INVALID_ARG, "k_caches / v_caches is NULL") : QWEN3_OK;
  if (capacity < need_rows)
    return fail(QWEN3_ERR_INVALID_ARG, "capacity (%d) must be >= %d", capacity, need_rows);
  for (int l = 0; l < cfg->n_layers; ++l) {
    if (!kc[l] || !vc[l] || kc[l] == vc[l])
      return fail(QWEN3_ERR_INVALID_ARG, "layer %d: caches must be two distinct non-NULL buffers", l);
    if (misaligned16({kc[l], vc[l]})) return fail(QWEN3_ERR_INVALID_ARG, "cache pointers must be 16-byte aligned");
  }
  return QWEN3_OK;
}

static int model_prefill_impl(const qwen3_model_cfg* cfg, const qwen3_model_weights* w, const int32_t* tokens,
                              int32_t seq_len, const int32_t* positions, const int32_t* ds_rows, int32_t n_ds,
                              const void* const* ds, void* const* k_caches, void* const* v_caches,
                              int32_t capacity, float* logits, void* workspace, size_t workspace_bytes,
                              void* stream) {
  if (!cfg) return fail(QWEN3_ERR_INVALID_ARG, "cfg is NULL");
  int st = check_cfg(&cfg->layer);
  if (st) return st;
  if (cfg->n_layers < 0) return fail(QWEN3_ERR_INVALID_ARG, "n_layers (%d) must be >= 0", cfg->n_layers);
  if (cfg->vocab < 1) return fail(QWEN3_ERR_INVALID_ARG, "vocab (%d) must be >= 1", cfg->vocab);
  if (cfg->n_deepstack_layers < 0 || cfg->n_deepstack_layers > cfg->n_layers)
    return fail(QWEN3_ERR_INVALID_ARG, "n_deepstack_layers (%d) must be in [0, n_layers = %d]",
                cfg->n_deepstack_layers, cfg->n_layers);
  if (seq_len < 1) return fail(QWEN3_ERR_INVALID_ARG, "seq_len must be >= 1 (got %d): empty prompt", seq_len);
  if (!tokens) return fail(QWEN3_ERR_INVALID_ARG, "tokens is NULL");
  if (!w || !w->token_embd || !w->output_norm || (cfg->n_layers > 0 && !w->layers))
    return fail(QWEN3_ERR_INVALID_ARG, "model weights (token_embd, output_norm, layers) must not be NULL");
  if (!positions || !logits) return fail(QWEN3_ERR_INVALID_ARG, "positions / logits is NULL");
  if (misaligned16({w->token_embd, w->output_norm, w->lm_head, logits}))
    return fail(QWEN3_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  const int nds = cfg->n_deepstack_layers;
  if ((st = check_ds_rows(ds_rows, n_ds, seq_len))) return st;
  if (n_ds > 0 && nds > 0) {
    if (!ds) return fail(QWEN3_ERR_INVALID_ARG, "n_ds = %d needs the slab array", n_ds);
    for (int l = 0; l < nds; ++l)
      if (!ds[l]) return fail(QWEN3_ERR_INVALID_ARG, "DeepStack slab %d is NULL", l);
  }
  for (int32_t i = 0; i < seq_len; ++i)
    if (tokens[i] < 0 || tokens[i] >= cfg->vocab)
      return fail(QWEN3_ERR_INVALID_ARG, "token id %d at position %d is outside [0, vocab = %d)", tokens[i], i,
                  cfg->vocab);
  const ModelWorkspace L = model_layout(cfg, seq_len);
  if (!workspace || workspace_bytes < L.total)
    return fail(QWEN3_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu%s)", L.total, workspace_bytes,
                workspace ? "" : ", NULL pointer");
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(QWEN3_ERR_WORKSPACE, "workspace must be 256-byte aligned");

  hipStream_t s = static_cast<hipStream_t>(stream);
  const int S = seq_len, H = cfg->layer.hidden;
  const qwen3_dtype wdt = plain_w(cfg->layer.wdtype);
  char* ws = static_cast<char*>(workspace);
  int32_t* tok = reinterpret_cast<int32_t*>(ws + L.tokens);
  float* x = reinterpret_cast<float*>(ws + L.x);
  float* xlast = reinterpret_cast<float*>(ws + L.xlast);
  hipError_t e = hipMemcpyAsync(tok, tokens, static_cast<size_t>(S) * 4, hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return hip_fail(e, "token upload");
  {
    KTimer t("embed_gather", s);
    e = q3::launch_embed_gather(tok, w->token_embd, wdt, x, S, H, s);
    if (e != hipSuccess) return hip_fail(e, "embed_gather launch");
  }
  const size_t lbytes = L.total - L.layer;
  for (int l = 0; l < cfg->n_layers; ++l) {
    const bool with_ds = l < nds && n_ds > 0;
    st = k_caches ? qwen3_layer_prefill_kv(&cfg->layer, &w->layers[l], x, x, S, positions,
                                           with_ds ? ds_rows : nullptr, with_ds ? n_ds : 0,
                                           with_ds ? ds[l] : nullptr, k_caches[l], v_caches[l], capacity,
                                           ws + L.layer, lbytes, stream)
                  : qwen3_layer_prefill(&cfg->layer, &w->layers[l], x, x, S, positions, with_ds ? ds_rows : nullptr,
                                        with_ds ? n_ds : 0, with_ds ? ds[l] : nullptr, ws + L.layer, lbytes, stream);
    if (st) return st;
  }
  if ((st = run_rmsnorm(x + static_cast<size_t>(S - 1) * H, w->output_norm, wdt, xlast, QWEN3_F32, 1, H,
                        cfg->layer.rms_eps, s)))
    return st;
  {
    KTimer t("lm_head", s);
    e = q3::launch_gemv_rows(w->lm_head ? w->lm_head : w->token_embd, wdt, xlast, logits, cfg->vocab, H, s);
    if (e != hipSuccess) return hip_fail(e, "lm_head launch");
  }
  return QWEN3_OK;
}

int qwen3_model_prefill_logits_last(const qwen3_model_cfg* cfg, const qwen3_model_weights* w,
                                    const int32_t* tokens, int32_t seq_len, const int32_t* positions,
                                    const int32_t* ds_rows, int32_t n_ds, const void* const* ds, float* logits,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  return model_prefill_impl(cfg, w, tokens, seq_len, positions, ds_rows, n_ds, ds, nullptr, nullptr, 0, logits,
                            workspace, workspace_bytes, stream);
}

int qwen3_model_prefill_logits_last_kv(const qwen3_model_cfg* cfg, const qwen3_model_weights* w,
                                       const int32_t* tokens, int32_t seq_len, const int32_t* positions,
                                       const int32_t* ds_rows, int32_t n_ds, const void* const* ds,
                                       void* const* k_caches, void* const* v_caches, int32_t capacity,
                                       float* logits, void* workspace, size_t workspace_bytes, void* stream) {
  if (!cfg) return fail(QWEN3_ERR_INVALID_ARG, "cfg is NULL");
  int st = check_model_caches(cfg, k_caches, v_caches, capacity, seq_len, true);
  if (st) return st;
  return model_prefill_impl(cfg, w, tokens, seq_len, positions, ds_rows, n_ds, ds, k_caches, v_caches, capacity,
                            logits, workspace, workspace_bytes, stream);
}

struct ModelDecodeWorkspace {
  size_t x, xlast, layer, total;
};

static ModelDecodeWorkspace model_decode_layout(const qwen3_model_cfg* c, int32_t capacity) {
  ModelDecodeWorkspace m{};
  const size_t H = c->layer.hidden;
  m.x = 0;
  m.xlast = m.x + align256(H * 4);
  m.layer = m.xlast + align256(H * 4);
  m.total = m.layer + qwen3_layer_decode_workspace_bytes(&c->layer, capacity);
  return m;
}

size_t qwen3_model_decode_workspace_bytes(const qwen3_model_cfg* cfg, int32_t capacity) {
  if (!cfg || capacity < 1 || cfg->n_layers < 0) return 0;
  const size_t layer = qwen3_layer_decode_workspace_bytes(&cfg->layer, capacity);
  if (layer == 0) return 0;
  return model_decode_layout(cfg, capacity).total;
}

int qwen3_model_decode_logits(const qwen3_model_cfg* cfg, const qwen3_model_weights* w, int32_t token,
                              const int32_t* position, void* const* k_caches, void* const* v_caches,
                              int32_t capacity, int32_t len, float* logits, void* workspace,
                              size_t workspace_bytes, void* stream) {
  int st = check_model(cfg, w, logits);
  if (st) return st;
  if (token < 0 || token >= cfg->vocab)
    return fail(QWEN3_ERR_INVALID_ARG, "token id %d is outside [0, vocab = %d)", token, cfg->vocab);
  if (!position) return fail(QWEN3_ERR_INVALID_ARG, "position is NULL");
  if (len < 0 || len >= capacity)
    return fail(QWEN3_ERR_INVALID_ARG, "len (%d) must be in [0, capacity = %d): the new token takes row len", len,
                capacity);
  if (cfg->n_layers > 0 && (st = check_model_caches(cfg, k_caches, v_caches, capacity, len + 1, true))) return st;
  const ModelDecodeWorkspace L = model_decode_layout(cfg, capacity);
  if (!workspace || workspace_bytes < L.total)
    return fail(QWEN3_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu%s)", L.total, workspace_bytes,
                workspace ? "" : ", NULL pointer");
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(QWEN3_ERR_WORKSPACE, "workspace must be 256-byte aligned");

  hipStream_t s = static_cast<hipStream_t>(stream);
  const int H = cfg->layer.hidden;
  const qwen3_dtype wdt = plain_w(cfg->layer.wdtype);
  char* ws = static_cast<char*>(workspace);
  float* x = reinterpret_cast<float*>(ws + L.x);
  float* xlast = reinterpret_cast<float*>(ws + L.xlast);
  hipError_t e;
  {
    KTimer t("embed_gather", s);
    e = q3::launch_embed_row(w->token_embd, wdt, token, x, H, s);
    if (e != hipSuccess) return hip_fail(e, "embed_row launch");
  }
  const size_t lbytes = L.total - L.layer;
  for (int l = 0; l < cfg->n_layers; ++l) {
    st = qwen3_layer_decode(&cfg->layer, &w->layers[l], x, x, position, k_caches[l], v_caches[l], capacity, len,
                            ws + L.layer, lbytes, stream);
    if (st) return st;
  }
  if ((st = run_rmsnorm(x, w->output_norm, wdt, xlast, QWEN3_F32, 1, H, cfg->layer.rms_eps, s))) return st;
  {
    KTimer t("lm_head", s);
    e = q3::launch_gemv_rows(w->lm_head ? w->lm_head : w->token_embd, wdt, xlast, logits, cfg->vocab, H, s);
    if (e != hipSuccess) return hip_fail(e, "lm_head launch");
  }
  return QWEN3_OK;
}

int qk_norm_mrope(void* q, void* k, int32_t seq_len, int32_t n_heads, int32_t n_kv_heads, int32_t head_dim,
                  const void* q_norm, const void* k_norm, float eps, const int32_t* positions, float theta,
                  const int32_t mrope_section[3], qwen3_dtype dtype, qwen3_dtype norm_dtype, void* stream) {
  if (!valid_dtype(dtype) || !valid_dtype(norm_dtype))
    return fail(QWEN3_ERR_INVALID_ARG, "dtype (%d, %d) is not a qwen3_dtype", dtype, norm_dtype);
  if (seq_len < 1) return fail(QWEN3_ERR_INVALID_ARG, "seq_len must be >= 1 (got %d)", seq_len);
  if (n_heads < 1 || n_kv_heads < 1)
    return fail(QWEN3_ERR_INVALID_ARG, "n_heads (%d) and n_kv_heads (%d) must be >= 1", n_heads, n_kv_heads);
  if (head_dim != 64 && head_dim != 128)
    return fail(QWEN3_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", head_dim);
  int st = check_sections(mrope_section, head_dim);
  if (st) return st;
  if (!q || !q_norm || !k || !k_norm || !positions) return fail(QWEN3_ERR_INVALID_ARG, "NULL tensor pointer");
  if (misaligned16({q, k, q_norm, k_norm}))
    return fail(QWEN3_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  if (!(eps >= 0.f) || !(theta > 1.f)) return fail(QWEN3_ERR_INVALID_ARG, "eps must be >= 0 and theta > 1");
  q3::RopeParams p{q, k, static_cast<int64_t>(n_heads) * head_dim, static_cast<int64_t>(n_kv_heads) * head_dim,
                   seq_len, n_heads, n_kv_heads, q_norm, k_norm, norm_dtype, positions, eps,
                   std::log2(static_cast<double>(theta)), mrope_section[1], mrope_section[2]};
  return run_qk_norm_mrope(p, head_dim, dtype, static_cast<hipStream_t>(stream));
}

static int attention_entry(const void* q, const void* k, const void* v, void* out, int32_t seq_len,
                           int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, float scale, qwen3_dtype dtype,
                           int causal, void* stream) {
  if (!valid_dtype(dtype)) return fail(QWEN3_ERR_INVALID_ARG, "dtype %d is not a qwen3_dtype", dtype);
  if (seq_len < 1) return fail(QWEN3_ERR_INVALID_ARG, "seq_len must be >= 1 (got %d)", seq_len);
  int st = check_heads(n_heads, n_kv_heads, head_dim, dtype);
  if (st) return st;
  if (!q || !k || !v || !out) return fail(QWEN3_ERR_INVALID_ARG, "NULL tensor pointer");
  if (misaligned16({q, k, v, out})) return fail(QWEN3_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(QWEN3_ERR_INVALID_ARG, "scale must be finite and > 0");
  return run_attention(q, k, v, out, static_cast<int64_t>(n_heads) * head_dim,
                       static_cast<int64_t>(n_kv_heads) * head_dim, static_cast<int64_t>(n_kv_heads) * head_dim,
                       static_cast<int64_t>(n_heads) * head_dim, seq_len, n_heads, n_kv_heads, head_dim, scale,
                       dtype, causal, static_cast<hipStream_t>(stream));
}

int gqa_causal_attention(const void* q, const void* k, const void* v, void* out, int32_t seq_len,
                         int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, float scale,
                         qwen3_dtype dtype, void* stream) {
  return attention_entry(q, k, v, out, seq_len, n_heads, n_kv_heads, head_dim, scale, dtype, 1, stream);
}

int gqa_bidirectional_attention(const void* q, const void* k, const void* v, void* out, int32_t seq_len,
                                int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, float scale,
                                qwen3_dtype dtype, void* stream) {
  return attention_entry(q, k, v, out, seq_len, n_heads, n_kv_heads, head_dim, scale, dtype, 0, stream);
}

int vision_rope_tables(int32_t frames, int32_t grid_h, int32_t grid_w, int32_t merge, int32_t head_dim,
                       float theta, int32_t layout, float* cos_out, float* sin_out, void* stream) {
  if (frames < 1 || grid_h < 1 || grid_w < 1 || merge < 1)
    return fail(QWEN3_ERR_INVALID_ARG, "grid (%d, %d, %d) and merge (%d) must be >= 1", frames, grid_h, grid_w,
                merge);
  if (grid_h % merge != 0 || grid_w % merge != 0)
    return fail(QWEN3_ERR_INVALID_ARG, "grid_h (%d) and grid_w (%d) must be multiples of merge (%d)", grid_h,
                grid_w, merge);
  if (layout != 0 && layout != 1) return fail(QWEN3_ERR_INVALID_ARG, "layout must be 0 (2-D) or 1 (3-axis)");
  if (head_dim < 4 || head_dim % (layout == 0 ? 4 : 32) != 0)
    return fail(QWEN3_ERR_INVALID_ARG, "head_dim (%d) must be a positive multiple of %d for layout %d", head_dim,
                layout == 0 ? 4 : 32, layout);
  if (!(theta > 1.f) || !std::isfinite(theta)) return fail(QWEN3_ERR_INVALID_ARG, "theta must be finite and > 1");
  if (!cos_out || !sin_out) return fail(QWEN3_ERR_INVALID_ARG, "NULL tensor pointer");
  if (misaligned16({cos_out, sin_out})) return fail(QWEN3_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  if (static_cast<int64_t>(frames) * grid_h * grid_w > 0x7fffffff / head_dim)
    return fail(QWEN3_ERR_UNSUPPORTED, "grid too large");
  hipStream_t s = static_cast<hipStream_t>(stream);
  KTimer t("vision_rope_tables", s);
  const hipError_t e = q3::launch_vision_rope_tables(layout, frames, grid_h, grid_w, merge, head_dim,
                                                     std::log2(static_cast<double>(theta)), cos_out, sin_out, s);
  return e == hipSuccess ? QWEN3_OK : hip_fail(e, "vision_rope_tables launch");
}

int apply_rope_tables(void* x, int32_t n, int32_t heads, int32_t head_dim, int64_t row_stride,
                      const float* cos_tab, const float* sin_tab, int32_t pairing, qwen3_dtype dtype,
                      void* stream) {
  if (!valid_dtype(dtype)) return fail(QWEN3_ERR_INVALID_ARG, "dtype %d is not a qwen3_dtype", dtype);
  if (n < 1 || heads < 1) return fail(QWEN3_ERR_INVALID_ARG, "n (%d) and heads (%d) must be >= 1", n, heads);
  if (head_dim < 2 || head_dim % 2 != 0) return fail(QWEN3_ERR_INVALID_ARG, "head_dim (%d) must be even", head_dim);
  if (row_stride < static_cast<int64_t>(heads) * head_dim)
    return fail(QWEN3_ERR_INVALID_ARG, "row_stride (%lld) must be >= heads * head_dim",
                static_cast<long long>(row_stride));
  if (pairing != 0 && pairing != 1) return fail(QWEN3_ERR_INVALID_ARG, "pairing must be 0 (split) or 1 (adjacent)");
  if (!x || !cos_tab || !sin_tab) return fail(QWEN3_ERR_INVALID_ARG, "NULL tensor pointer");
  if (misaligned16({x, cos_tab, sin_tab})) return fail(QWEN3_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  KTimer t("apply_rope_tables", s);
  const hipError_t e = q3::launch_apply_rope_tables(x, dtype, n, heads, head_dim, row_stride, cos_tab, sin_tab,
                                                    pairing, s);
  return e == hipSuccess ? QWEN3_OK : hip_fail(e, "apply_rope_tables launch");
}

int swiglu_ffn(const void* x_normed, const void* w_gate, const void* w_up, const void* w_down,
               const void* residual, void* out, int32_t seq_len, int32_t hidden, int32_t ffn,
               qwen3_dtype wdtype, qwen3_dtype x_dtype, qwen3_dtype out_dtype, void* workspace,
               size_t workspace_bytes, void* stream) {
  int st = check_formats(wdtype, x_dtype);
  if (st) return st;
  if (!valid_dtype(out_dtype)) return fail(QWEN3_ERR_INVALID_ARG, "out_dtype %d is not a qwen3_dtype", out_dtype);
  if (seq_len < 1) return fail(QWEN3_ERR_INVALID_ARG, "seq_len must be >= 1 (got %d)", seq_len);
  if (hidden < 256 || hidden % 256 != 0)
    return fail(QWEN3_ERR_UNSUPPORTED, "hidden (%d) must be a positive multiple of 256", hidden);
  if (ffn < 128 || ffn % 128 != 0) return fail(QWEN3_ERR_UNSUPPORTED, "ffn (%d) must be a positive multiple of 128", ffn);
  if (!x_normed || !w_gate || !w_up || !w_down || !out) return fail(QWEN3_ERR_INVALID_ARG, "NULL tensor pointer");
  if (misaligned16({x_normed, w_gate, w_up, w_down, residual, out, workspace}))
    return fail(QWEN3_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  if (out_dtype != QWEN3_F32 && (residual || out_dtype != x_dtype))
    return fail(QWEN3_ERR_UNSUPPORTED, "a 16-bit output must have x_dtype and no residual");
  const size_t need = swiglu_ffn_workspace_bytes(seq_len, ffn, x_dtype);
  if (!workspace || workspace_bytes < need)
    return fail(QWEN3_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", need, workspace_bytes);
  return run_ffn(x_normed, w_gate, w_up, w_down, static_cast<const float*>(residual), out, out_dtype,
                 workspace, seq_len, hidden, ffn, wdtype, x_dtype, static_cast<hipStream_t>(stream));
}

int qwen3_tile_weights(const void* src, qwen3_dtype src_dtype, int32_t rows, int32_t cols, void* dst, void* stream) {
  if (!valid_dtype(src_dtype)) return fail(QWEN3_ERR_INVALID_ARG, "src_dtype %d is not an element type", src_dtype);
  if (!src || !dst) return fail(QWEN3_ERR_INVALID_ARG, "src / dst is NULL");
  if (misaligned16({src, dst})) return fail(QWEN3_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  if (rows < 16 || rows % 16 != 0 || cols < 32 || cols % 32 != 0)
    return fail(QWEN3_ERR_UNSUPPORTED, "rows (%d) must be a positive multiple of 16 and cols (%d) of 32", rows, cols);
  {
    const size_t n = static_cast<size_t>(rows) * cols;
    const char* a = static_cast<const char*>(src);
    const char* b = static_cast<const char*>(dst);
    if (a < b + 2 * n && b < a + n * dsize(src_dtype)) return fail(QWEN3_ERR_INVALID_ARG, "dst overlaps src");
  }
  KTimer t("tile_weights", static_cast<hipStream_t>(stream));
  const hipError_t e = q3::launch_tile_matrix(src, src_dtype, rows, cols, static_cast<uint16_t*>(dst),
                                              static_cast<hipStream_t>(stream));
  return e == hipSuccess ? QWEN3_OK : hip_fail(e, "tile_weights launch");
}

int rms_norm_rows(const float* x, const void* w, void* y, int32_t rows, int32_t hidden, float eps,
                  qwen3_dtype w_dtype, qwen3_dtype y_dtype, void* stream) {
  if (!valid_dtype(w_dtype) || !valid_dtype(y_dtype)) return fail(QWEN3_ERR_INVALID_ARG, "bad dtype");
  if (rows < 1) return fail(QWEN3_ERR_INVALID_ARG, "rows must be >= 1 (got %d)", rows);
  if (hidden < 256 || hidden % 256 != 0 || hidden > 16384)
    return fail(QWEN3_ERR_UNSUPPORTED, "hidden (%d) must be a multiple of 256 in [256, 16384]", hidden);
  if (!x || !w || !y) return fail(QWEN3_ERR_INVALID_ARG, "NULL tensor pointer");
  if (misaligned16({x, w, y})) return fail(QWEN3_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  if (!(eps >= 0.f)) return fail(QWEN3_ERR_INVALID_ARG, "eps must be >= 0");
  return run_rmsnorm(x, w, w_dtype, y, y_dtype, rows, hidden, eps, static_cast<hipStream_t>(stream));
}

int qwen3_timing_enable(int enable) {
  std::lock_guard<std::mutex> lk(g_tmu);
  g_timing = enable != 0;
  return QWEN3_OK;
}

int qwen3_timing_collect(qwen3_kernel_time* out, int32_t max_entries, int32_t* n_out) {
  std::lock_guard<std::mutex> lk(g_tmu);
  std::map<std::string, std::pair<int, double>> agg;
  std::map<std::string, std::vector<float>> each;  // every launch's time, for the median
  std::vector<std::string> order;
  for (int i = 0; i < g_used; ++i) {
    hipError_t e = hipEventSynchronize(g_events[2 * i + 1]);
    if (e != hipSuccess) {
      g_used = 0;
      return hip_fail(e, "timing event synchronize");
    }
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, g_events[2 * i], g_events[2 * i + 1]);
    if (e != hipSuccess) {
      g_used = 0;
      return hip_fail(e, "timing elapsed time");
    }
    const std::string name = g_slot_name[i];
    if (!agg.count(name)) order.push_back(name);
    agg[name].first += 1;
    agg[name].second += ms;
    each[name].push_back(ms);
  }
  g_used = 0;
  int n = 0;
  for (const auto& name : order) {
    if (n >= max_entries) break;
    if (out) {
      std::memset(&out[n], 0, sizeof(out[n]));
      std::strncpy(out[n].name, name.c_str(), sizeof(out[n].name) - 1);
      out[n].launches = agg[name].first;
      out[n].total_ms = agg[name].second;
      std::vector<float>& v = each[name];
      std::sort(v.begin(), v.end());
      const size_t h = v.size() / 2;
      out[n].median_ms = v.size() % 2 ? v[h] : 0.5 * (static_cast<double>(v[h - 1]) + v[h]);
    }
    ++n;
  }
  if (n_out) *n_out = n;
  return QWEN3_OK;
}

// ---- KV cache and one decode step ---------------------------------------------------------
int kv_cache_write(const void* k, const void* v, int64_t k_stride, int64_t v_stride, int32_t n, int32_t n_kv_heads,
                   int32_t head_dim, qwen3_dtype src_dtype, void* k_cache, void* v_cache, qwen3_dtype cache_dtype,
                   int32_t capacity, int32_t row0, void* stream) {
  if (!valid_dtype(src_dtype) || !valid_dtype(cache_dtype))
    return fail(QWEN3_ERR_INVALID_ARG, "src_dtype / cache_dtype is not a qwen3_dtype");
  if (n < 1 || n_kv_heads < 1) return fail(QWEN3_ERR_INVALID_ARG, "n (%d) and n_kv_heads (%d) must be >= 1", n, n_kv_heads);
  if (head_dim < 8 || head_dim % 8 != 0)
    return fail(QWEN3_ERR_UNSUPPORTED, "head_dim (%d) must be a positive multiple of 8", head_dim);
  if (k_stride < static_cast<int64_t>(n_kv_heads) * head_dim || v_stride < static_cast<int64_t>(n_kv_heads) * head_dim ||
      k_stride % 8 != 0 || v_stride % 8 != 0)
    return fail(QWEN3_ERR_INVALID_ARG, "row strides must be multiples of 8 and >= n_kv_heads * head_dim");
  if (row0 < 0 || capacity < 1 || static_cast<int64_t>(row0) + n > capacity)
    return fail(QWEN3_ERR_INVALID_ARG, "rows [%d, %lld) do not fit a capacity of %d", row0,
                static_cast<long long>(row0) + n, capacity);
  if (!k || !v || !k_cache || !v_cache) return fail(QWEN3_ERR_INVALID_ARG, "NULL tensor pointer");
  if (misaligned16({k, v, k_cache, v_cache})) return fail(QWEN3_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  KTimer t("kv_cache_write", s);
  q3::KvWriteParams p{k, v, k_stride, v_stride, n, n_kv_heads, head_dim, k_cache, v_cache, capacity, row0};
  const hipError_t e = q3::launch_kv_cache_write(p, src_dtype, cache_dtype, s);
  return e == hipSuccess ? QWEN3_OK : hip_fail(e, "kv_cache_write launch");
}

static size_t decode_attn_scratch(int32_t nh, int32_t nkv, int32_t hd, int32_t max_len, size_t* o_bytes) {
  const size_t ns = static_cast<size_t>(q3::decode_max_splits(max_len, nkv));
  *o_bytes = align256(static_cast<size_t>(nh) * ns * hd * 4);
  return *o_bytes + align256(static_cast<size_t>(nh) * ns * 2 * 4);
}

static int check_decode_heads(int32_t nh, int32_t nkv, int32_t hd) {
  if (nh < 1 || nkv < 1 || nh % nkv != 0)
    return fail(QWEN3_ERR_INVALID_ARG, "n_heads (%d) must be a positive multiple of n_kv_heads (%d)", nh, nkv);
  if (nh / nkv > 16) return fail(QWEN3_ERR_UNSUPPORTED, "n_heads / n_kv_heads must be <= 16 (got %d)", nh / nkv);
  if (hd != 64 && hd != 128) return fail(QWEN3_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", hd);
  return QWEN3_OK;
}

static int run_decode_attention(const float* q, const void* kc, const void* vc, int32_t capacity, int32_t len,
                                int32_t nh, int32_t nkv, int32_t hd, float scale, qwen3_dtype cdt, float* out,
                                char* scratch, hipStream_t s) {
  size_t ob;
  (void)decode_attn_scratch(nh, nkv, hd, len, &ob);
  q3::DecodeAttnParams p{q, kc, vc, capacity, len, nh, nkv, scale * 1.4426950408889634f,
                         q3::decode_tiles_per_split(len, nkv), q3::decode_num_splits(len, nkv),
                         reinterpret_cast<float*>(scratch), reinterpret_cast<float*>(scratch + ob)};
  KTimer t("decode_attention", s);
  const hipError_t e = q3::launch_decode_attention(p, hd, cdt, out, s);
  return e == hipSuccess ? QWEN3_OK : hip_fail(e, "decode_attention launch");
}

size_t gqa_decode_attention_workspace_bytes(int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, int32_t len) {
  if (n_heads < 1 || n_kv_heads < 1 || n_heads % n_kv_heads != 0 || head_dim < 1 || len < 1) return 0;
  size_t ob;
  return decode_attn_scratch(n_heads, n_kv_heads, head_dim, len, &ob);
}

int gqa_decode_attention(const float* q, const void* k_cache, const void* v_cache, int32_t capacity, int32_t len,
                         int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, float scale, qwen3_dtype cache_dtype,
                         float* out, void* workspace, size_t workspace_bytes, void* stream) {
  if (!valid_dtype(cache_dtype)) return fail(QWEN3_ERR_INVALID_ARG, "cache_dtype %d is not a qwen3_dtype", cache_dtype);
  int st = check_decode_heads(n_heads, n_kv_heads, head_dim);
  if (st) return st;
  if (len < 1 || len > capacity)
    return fail(QWEN3_ERR_INVALID_ARG, "len (%d) must be in [1, capacity = %d]", len, capacity);
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(QWEN3_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (!q || !k_cache || !v_cache || !out) return fail(QWEN3_ERR_INVALID_ARG, "NULL tensor pointer");
  if (misaligned16({q, k_cache, v_cache, out})) return fail(QWEN3_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  const size_t need = gqa_decode_attention_workspace_bytes(n_heads, n_kv_heads, head_dim, len);
  if (!workspace || workspace_bytes < need)
    return fail(QWEN3_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu%s)", need, workspace_bytes,
                workspace ? "" : ", NULL pointer");
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(QWEN3_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  return run_decode_attention(q, k_cache, v_cache, capacity, len, n_heads, n_kv_heads, head_dim, scale, cache_dtype,
                              out, static_cast<char*>(workspace), static_cast<hipStream_t>(stream));
}

struct DecodeWorkspace {
  size_t xn, qkv, o, act, attn, total;
};

static DecodeWorkspace decode_layout(const qwen3_layer_cfg* c, int32_t capacity) {
  const size_t q_dim = static_cast<size_t>(c->n_heads) * c->head_dim;
  const size_t kv_dim = static_cast<size_t>(c->n_kv_heads) * c->head_dim;
  DecodeWorkspace d;
  size_t ob;
  d.xn = 0;
  d.qkv = d.xn + align256(static_cast<size_t>(c->hidden) * 4);
  d.o = d.qkv + align256((q_dim + 2 * kv_dim) * 4);
  d.act = d.o + align256(q_dim * 4);
  d.attn = d.act + align256(static_cast<size_t>(c->ffn) * 4);
  d.total = d.attn + decode_attn_scratch(c->n_heads, c->n_kv_heads, c->head_dim, capacity, &ob);
  return d;
}

size_t qwen3_layer_decode_workspace_bytes(const qwen3_layer_cfg* cfg, int32_t capacity) {
  if (!cfg || capacity < 1 || cfg->n_heads < 1 || cfg->n_kv_heads < 1 || cfg->n_heads % cfg->n_kv_heads != 0)
    return 0;
  return decode_layout(cfg, capacity).total;
}

// One matrix-vector product group: p's W0..W2 come from m (n matrices). Dense matrices use the
// dense kernel; quantized ones of one format the quantized kernel; a store group whose matrices
// differ in format runs one launch per matrix.
static int run_gemv(const char* name, const MatW* const* m, int n, q3::GemvParams p, int epi, qwen3_dtype wdt,
                    hipStream_t s) {
  KTimer t(name, s);
  bool same = true;
  for (int i = 1; i < n; ++i) same = same && m[i]->fmt == m[0]->fmt;
  hipError_t e = hipSuccess;
  if (same) {
    p.W0 = m[0]->data;
    p.W1 = n > 1 ? m[1]->data : nullptr;
    p.W2 = n > 2 ? m[2]->data : nullptr;
    if (m[0]->fmt == QWEN3_W_DENSE) e = q3::launch_gemv(p, epi, wdt, s);
    else e = q3::launch_gemv_quant(p, epi, m[0]->fmt, m[0]->rs, n > 1 ? m[1]->rs : nullptr, n > 2 ? m[2]->rs : nullptr, s);
  } else {
    if (epi != q3::GV_STORE) return fail(QWEN3_ERR_UNSUPPORTED, "%s: mixed weight formats", name);
    const int lo[3] = {0, p.nseg0, p.nseg1}, hi[3] = {p.nseg0, p.nseg1, p.rows};
    for (int i = 0; i < n && e == hipSuccess; ++i) {
      q3::GemvParams q = p;
      q.W0 = m[i]->data;
      q.W1 = q.W2 = nullptr;
      q.rows = hi[i] - lo[i];
      q.nseg0 = q.nseg1 = q.rows;
      q.y = p.y + lo[i];
      if (m[i]->fmt == QWEN3_W_DENSE) e = q3::launch_gemv(q, epi, wdt, s);
      else e = q3::launch_gemv_quant(q, epi, m[i]->fmt, m[i]->rs, nullptr, nullptr, s);
    }
  }
  return e == hipSuccess ? QWEN3_OK : hip_fail(e, name);
}

static int layer_decode_impl(const qwen3_layer_cfg* cfg, const LayerW& w, const float* x_in, float* x_out,
                             const int32_t* position, void* k_cache, void* v_cache, int32_t capacity, int32_t len,
                             void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_cfg(cfg);
  if (st) return st;
  if ((st = check_decode_heads(cfg->n_heads, cfg->n_kv_heads, cfg->head_dim))) return st;
  bool quant = false;
  if ((st = check_layer_w(w, cfg, &quant))) return st;
  if (!x_in || !x_out || !position || !k_cache || !v_cache)
    return fail(QWEN3_ERR_INVALID_ARG, "x_in / x_out / position / k_cache / v_cache is NULL");
  if (k_cache == v_cache) return fail(QWEN3_ERR_INVALID_ARG, "k_cache and v_cache must be different buffers");
  if (misaligned16({x_in, x_out, k_cache, v_cache}))
    return fail(QWEN3_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  if (len < 0 || len >= capacity)
    return fail(QWEN3_ERR_INVALID_ARG, "len (%d) must be in [0, capacity = %d): the new token takes row len", len,
                capacity);
  {
    const size_t xb = static_cast<size_t>(cfg->hidden) * 4;
    const char* a = reinterpret_cast<const char*>(x_in);
    const char* b = reinterpret_cast<const char*>(x_out);
    if (a != b && a < b + xb && b < a + xb)
      return fail(QWEN3_ERR_INVALID_ARG, "x_out partially overlaps x_in (only x_out == x_in is allowed)");
  }
  const DecodeWorkspace L = decode_layout(cfg, capacity);
  if (!workspace || workspace_bytes < L.total)
    return fail(QWEN3_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu%s)", L.total, workspace_bytes,
                workspace ? "" : ", NULL pointer");
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(QWEN3_ERR_WORKSPACE, "workspace must be 256-byte aligned");

  hipStream_t s = static_cast<hipStream_t>(stream);
  const qwen3_dtype wdt = plain_w(cfg->wdtype), cdt = cfg->act_dtype;
  const int wt = cfg->wdtype == QWEN3_F16_TILED;   // dense matrices tiled (quantized ones never are)
  const int H = cfg->hidden, nh = cfg->n_heads, nkv = cfg->n_kv_heads, hd = cfg->head_dim, F = cfg->ffn;
  const int q_dim = nh * hd, kv_dim = nkv * hd, qkv_dim = q_dim + 2 * kv_dim;
  char* ws = static_cast<char*>(workspace);
  float* xn = reinterpret_cast<float*>(ws + L.xn);
  float* qkv = reinterpret_cast<float*>(ws + L.qkv);
  float* o = reinterpret_cast<float*>(ws + L.o);
  float* act = reinterpret_cast<float*>(ws + L.act);

  // input RMSNorm of the new row: folded into the q | k | v product for dense weights (the
  // product runs on x * attn_norm and is scaled by 1/rms), a separate fp32 row otherwise
  const bool fold_norm = !quant;
  if (!fold_norm && (st = run_rmsnorm(x_in, w.attn_norm, wdt, xn, QWEN3_F32, 1, H, cfg->rms_eps, s))) return st;
  // q | k | v of the new token
  {
    const MatW* g[3] = {&w.wq, &w.wk, &w.wv};
    q3::GemvParams p{nullptr, nullptr, nullptr, q_dim, q_dim + kv_dim, fold_norm ? x_in : xn, qkv, nullptr,
                     qkv_dim, H};
    p.w_tiled = wt;
    if (fold_norm) {
      p.norm_w = w.attn_norm;
      p.norm_dt = wdt;
      p.eps = cfg->rms_eps;
    }
    if ((st = run_gemv("gemv_qkv", g, 3, p, q3::GV_STORE, wdt, s))) return st;
  }
  // per-head RMSNorm + interleaved MRoPE at the token's position; the same launch appends k'
  // and v at row len of the caches
  {
    q3::RopeParams p{qkv, qkv + q_dim, qkv_dim, qkv_dim, 1, nh, nkv, w.q_norm, w.k_norm, wdt, position,
                     cfg->rms_eps, std::log2(static_cast<double>(cfg->rope_theta)), cfg->mrope_section[1],
                     cfg->mrope_section[2]};
    p.kc = k_cache;
    p.vc = v_cache;
    p.v = qkv + q_dim + kv_dim;
    p.v_stride = qkv_dim;
    p.capacity = capacity;
    p.row0 = len;
    p.cache_dt = cdt;
    if ((st = run_qk_norm_mrope(p, hd, QWEN3_F32, s))) return st;
  }
  // the new query over the len + 1 cached keys
  if ((st = run_decode_attention(qkv, k_cache, v_cache, capacity, len + 1, nh, nkv, hd,
                                 1.0f / std::sqrt(static_cast<float>(hd)), cdt, o, ws + L.attn, s)))
    return st;
  // y1 = x + o Wo^T
  {
    const MatW* g[1] = {&w.wo};
    q3::GemvParams p{nullptr, nullptr, nullptr, H, H, o, x_out, x_in, H, q_dim};
    p.w_tiled = wt;
    if ((st = run_gemv("gemv_o_resid", g, 1, p, q3::GV_RESID, wdt, s))) return st;
  }
  if (!fold_norm && (st = run_rmsnorm(x_out, w.ffn_norm, wdt, xn, QWEN3_F32, 1, H, cfg->rms_eps, s))) return st;
  {
    const MatW* g[2] = {&w.wg, &w.wu};
    q3::GemvParams p{nullptr, nullptr, nullptr, F, F, fold_norm ? x_out : xn, act, nullptr, F, H};
    p.w_tiled = wt;
    if (fold_norm) {
      p.norm_w = w.ffn_norm;
      p.norm_dt = wdt;
      p.eps = cfg->rms_eps;
    }
    if ((st = run_gemv("gemv_gate_up_swiglu", g, 2, p, q3::GV_SWIGLU, wdt, s))) return st;
  }
  {
    const MatW* g[1] = {&w.wd};
    q3::GemvParams p{nullptr, nullptr, nullptr, H, H, act, x_out, x_out, H, F};
    p.w_tiled = wt;
    if ((st = run_gemv("gemv_down_resid", g, 1, p, q3::GV_RESID, wdt, s))) return st;
  }
  return QWEN3_OK;
}

int qwen3_layer_decode(const qwen3_layer_cfg* cfg, const qwen3_layer_weights* w, const float* x_in, float* x_out,
                       const int32_t* position, void* k_cache, void* v_cache, int32_t capacity, int32_t len,
                       void* workspace, size_t workspace_bytes, void* stream) {
  if (!w) return fail(QWEN3_ERR_INVALID_ARG, "weights is NULL");
  return layer_decode_impl(cfg, dense_layer(w), x_in, x_out, position, k_cache, v_cache, capacity, len, workspace,
                           workspace_bytes, stream);
}

int qwen3_layer_decode_quant(const qwen3_layer_cfg* cfg, const qwen3_layer_qweights* w, const float* x_in,
                             float* x_out, const int32_t* position, void* k_cache, void* v_cache, int32_t capacity,
                             int32_t len, void* workspace, size_t workspace_bytes, void* stream) {
  if (!w) return fail(QWEN3_ERR_INVALID_ARG, "weights is NULL");
  return layer_decode_impl(cfg, quant_layer(w), x_in, x_out, position, k_cache, v_cache, capacity, len, workspace,
                           workspace_bytes, stream);
}

}  // extern "C"
