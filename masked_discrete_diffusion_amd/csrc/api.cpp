// Host side of the C ABI declared in include/mdm_sparse.h: argument and
// capacity validation, workspace layout, cache-length bookkeeping, launches.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/mdm_sparse.h"
#include "common.hpp"
#include "kernels.hpp"

using namespace mdm;

namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxRegisters = 256;
constexpr int kMaxSelectCand = 1024;

thread_local std::string g_last_error;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct Layout {
  size_t err, rope_cos, rope_sin, ktab, qtab, qbuf, mvt, rvt, apart_o, apart_ml, hhi, hlo, partials, zpart, wt,
      total;
  int ktab_rows, r_pad;
  size_t zpart_bytes;
  int m_pad, n_vt, v_pad;
  bool wt_on;               // the tiled copy of W is kept (bf16, large vocabularies)
};

bool config_ok(const mdm_config* c, std::string* why) {
  auto fail = [&](const char* m) { if (why) *why = m; return false; };
  if (!c) return fail("config is NULL");
  if (c->batch <= 0 || c->n_heads <= 0 || c->n_kv_heads <= 0) return fail("batch and head counts must be positive");
  if (c->n_heads % c->n_kv_heads) return fail("n_heads must be a multiple of n_kv_heads");
  if (c->vocab <= 0 || c->seq_len <= 0) return fail("vocab and seq_len must be positive");
  if (c->n_registers < 0 || c->n_registers > kMaxRegisters) return fail("n_registers out of range");
  if (c->max_decode <= 0 || c->max_decode > c->seq_len) return fail("max_decode out of range");
  if (c->precision == MDM_BF16 && c->max_decode > kAttnMaxDecode) return fail("max_decode above 2048 (bf16)");
  if (c->precision != MDM_BF16 && c->precision != MDM_FP32) return fail("unknown precision");
  if (!(c->rope_theta > 1.0) || !std::isfinite(c->rope_theta)) return fail("rope_theta must be finite and > 1");
  return true;
}

bool shape_supported(const mdm_config* c, std::string* why) {
  if (c->head_dim != 64 && c->head_dim != 128) { if (why) *why = "head_dim must be 64 or 128"; return false; }
  const int64_t hidden = (int64_t)c->n_heads * c->head_dim;
  if (hidden % 64) { if (why) *why = "n_heads * head_dim must be a multiple of 64"; return false; }
  if (hidden > 8192) { if (why) *why = "n_heads * head_dim above 8192"; return false; }
  if ((int64_t)c->vocab + 1 + c->n_registers > INT32_MAX / 2) { if (why) *why = "vocab too large"; return false; }
  return true;
}

size_t slots_of(const mdm_config* c) { return align_up((size_t)c->seq_len, kKeyTile); }

Layout layout_of(const mdm_config* c) {
  Layout L{};
  const int hidden = c->n_heads * c->head_dim;
  const size_t max_pos = (size_t)c->seq_len + c->n_registers;
  L.n_vt = (c->vocab + kVocabTile - 1) / kVocabTile;
  L.v_pad = L.n_vt * kVocabTile;
  L.m_pad = (int)align_up((size_t)c->batch * c->max_decode, 128);
  size_t off = 0;
  L.err = off; off += kAlign;
  L.rope_cos = off; off = align_up(off + max_pos * (c->head_dim / 2) * sizeof(float), kAlign);
  L.rope_sin = off; off = align_up(off + max_pos * (c->head_dim / 2) * sizeof(float), kAlign);
  const bool bf16 = c->precision == MDM_BF16;
  const size_t esz = bf16 ? 2 : 4;
  // keys of the mask token at every position, then of the registers, per kv
  // head; rows up to seq_len + r_pad so whole register tiles stay in bounds
  L.r_pad = (int)align_up((size_t)std::max(c->n_registers, 1), kKeyTile);
  L.ktab_rows = c->seq_len + L.r_pad;
  L.ktab = off; off = align_up(off + (size_t)c->n_kv_heads * L.ktab_rows * c->head_dim * esz, kAlign);
  // bf16 attention: RoPE'd queries of the mask token at every position and of
  // the registers (same rows as the key table, all H heads), and of the rows
  // of the latest append (D rows of the next step)
  L.qtab = off; off = align_up(off + (bf16 ? (size_t)c->n_heads * L.ktab_rows * c->head_dim * esz : 0), kAlign);
  L.qbuf = off;
  off = align_up(off + (bf16 ? (size_t)c->batch * c->n_heads * c->max_decode * c->head_dim * esz : 0), kAlign);
  // bf16 attention: value tables of the transient keys, key-split partials
  const size_t kvd = (size_t)c->n_kv_heads * c->head_dim;
  L.mvt = off; off = align_up(off + (bf16 ? kvd * 8 * sizeof(uint16_t) : 0), kAlign);
  L.rvt = off; off = align_up(off + (bf16 ? kvd * L.r_pad * sizeof(uint16_t) : 0), kAlign);
  const size_t slots_rows = (size_t)kAttnSplitBlocks * 8 * 32;
  L.apart_o = off; off = align_up(off + (bf16 ? slots_rows * c->head_dim * sizeof(float) : 0), kAlign);
  L.apart_ml = off; off = align_up(off + (bf16 ? slots_rows * 2 * sizeof(float) : 0), kAlign);
  const size_t hbytes = bf16 ? (size_t)L.m_pad * hidden * sizeof(uint16_t) : 0;
  L.hhi = off; off = align_up(off + hbytes, kAlign);
  L.hlo = off; off = align_up(off + ((bf16 && c->accurate_conf) ? hbytes : 0), kAlign);
  // per (row, vocabulary tile) partial records; tiles are at least 32 columns
  L.partials = off; off = align_up(off + (size_t)L.m_pad * ((c->vocab + 31) / 32) * 8 * sizeof(float), kAlign);
  // split-hidden partial logits: at most 8 splits, capped at 32 MiB (splitting
  // is only chosen when few vocab tiles exist, i.e. for small vocabularies)
  const size_t zfull = 8 * (size_t)c->batch * c->max_decode * L.v_pad * sizeof(float);
  L.zpart_bytes = bf16 ? std::min(zfull, (size_t)32 << 20) : 0;
  L.zpart = off; off = align_up(off + L.zpart_bytes, kAlign);
  // bf16: the vocabulary head tiled for the screens' operand stream (built at init)
  L.wt_on = bf16 && c->vocab >= kTiledWMinVocab;
  L.wt = off; off = align_up(off + (L.wt_on ? tiled_w_elems(c->vocab, hidden) * sizeof(uint16_t) : 0), kAlign);
  L.total = off;
  return L;
}

}  // namespace

namespace {

constexpr int kMaxLayers = 16;

// Workspace of the upper layers (one region, reused by every layer in turn).
struct UpperLayout {
  size_t hhi, hlo, z, qbuf, tk, tvt, total;
  int m_cap, n_pad, q_rows, t_pad;
};

UpperLayout upper_layout_of(const mdm_config* c) {
  UpperLayout U{};
  const int hidden = c->n_heads * c->head_dim;
  const int n_proj = (c->n_heads + 2 * c->n_kv_heads) * c->head_dim;
  U.q_rows = c->seq_len + c->n_registers;                  // rows of one call: the prompt at most, + R
  U.m_cap = (int)align_up((size_t)c->batch * U.q_rows, 128);
  U.n_pad = (int)align_up((size_t)n_proj, kVocabTile);
  U.t_pad = (int)align_up((size_t)c->max_decode + c->n_registers, kKeyTile);
  size_t off = 0;
  U.hhi = off; off = align_up(off + (size_t)U.m_cap * hidden * 2, kAlign);
  U.hlo = off; off = align_up(off + (size_t)U.m_cap * hidden * 2, kAlign);
  U.z = off; off = align_up(off + (size_t)U.m_cap * U.n_pad * 4, kAlign);
  U.qbuf = off; off = align_up(off + (size_t)c->batch * c->n_heads * U.q_rows * c->head_dim * 2, kAlign);
  const size_t tb = (size_t)c->batch * c->n_kv_heads * U.t_pad * c->head_dim * 2;
  U.tk = off; off = align_up(off + tb, kAlign);
  U.tvt = off; off = align_up(off + tb, kAlign);
  U.total = off;
  return U;
}

}  // namespace

struct mdm_ctx {
  mdm_config cfg;
  mdm_buffers buf;
  hipStream_t stream;
  Geometry g;
  Layout L;
  int len;
  int q_rows;     // rows of the latest append whose queries are in the workspace, or -1
  float* trace = nullptr;   // per-row decision certificate (mdm_set_decision_trace), or NULL
  std::string err;
  // upper layers (mdm_attach_upper_layers)
  bool has_upper = false;
  mdm_upper_layers up{};
  UpperLayout U{};
  int len_up[kMaxLayers + 1] = {};
  int proj_nd[kMaxLayers + 1] = {};     // rows of the layer's latest projection (D, C), -1 if none
  int proj_nc[kMaxLayers + 1] = {};
  char* ws() const { return static_cast<char*>(buf.workspace); }
  char* uws() const { return static_cast<char*>(up.workspace); }
};

namespace {

mdm_status fail(mdm_ctx* ctx, mdm_status st, const char* fmt, ...) {
  char msg[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(msg, sizeof msg, fmt, ap);
  va_end(ap);
  if (ctx) ctx->err = msg;
  g_last_error = msg;
  return st;
}

mdm_status hip_check(mdm_ctx* ctx, hipError_t e, const char* what) {
  if (e == hipSuccess) return MDM_OK;
  return fail(ctx, MDM_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

// The first 256 bytes of the workspace: the error flag word, the decision
// counters (3 x uint32 at byte 64) and max_v ||W_v||_2 (float at byte 128).
int* err_word(mdm_ctx* c) { return reinterpret_cast<int*>(c->ws() + c->L.err); }
unsigned* decision_stats(mdm_ctx* c) { return reinterpret_cast<unsigned*>(c->ws() + c->L.err + 64); }
float* wmax_word(mdm_ctx* c) { return reinterpret_cast<float*>(c->ws() + c->L.err + 128); }
const float* rope_cos(mdm_ctx* c) { return reinterpret_cast<const float*>(c->ws() + c->L.rope_cos); }
const float* rope_sin(mdm_ctx* c) { return reinterpret_cast<const float*>(c->ws() + c->L.rope_sin); }

}  // namespace

extern "C" {

size_t mdm_cache_slots(const mdm_config* cfg) {
  if (!config_ok(cfg, nullptr) || !shape_supported(cfg, nullptr)) return 0;
  return slots_of(cfg);
}

size_t mdm_workspace_bytes(const mdm_config* cfg) {
  if (!config_ok(cfg, nullptr) || !shape_supported(cfg, nullptr)) return 0;
  return layout_of(cfg).total;
}

size_t mdm_element_bytes(const mdm_config* cfg) {
  if (!config_ok(cfg, nullptr)) return 0;
  return cfg->precision == MDM_BF16 ? 2 : 4;
}

mdm_status mdm_sparse_step_init(mdm_ctx** out, const mdm_config* cfg, const mdm_buffers* buf, void* stream) {
  if (!out) return fail(nullptr, MDM_E_ARG, "ctx out-pointer is NULL");
  *out = nullptr;
  std::string why;
  if (!config_ok(cfg, &why)) return fail(nullptr, MDM_E_ARG, "invalid config: %s", why.c_str());
  if (!shape_supported(cfg, &why)) return fail(nullptr, MDM_E_UNSUPPORTED, "unsupported shape: %s", why.c_str());
  if (!buf) return fail(nullptr, MDM_E_ARG, "buffers are NULL");
  if (!buf->tq || !buf->tk || !buf->tv || !buf->w_vocab || !buf->k_cache || !buf->v_cache ||
      !buf->cache_pos || !buf->cache_tok || !buf->workspace)
    return fail(nullptr, MDM_E_ARG, "a required buffer pointer is NULL");
  const Layout L = layout_of(cfg);
  if (buf->workspace_bytes < L.total)
    return fail(nullptr, MDM_E_SHAPE, "workspace has %zu bytes, needs %zu", buf->workspace_bytes, L.total);
  if (reinterpret_cast<uintptr_t>(buf->workspace) % kAlign)
    return fail(nullptr, MDM_E_ARG, "workspace must be 256-byte aligned");
  const uintptr_t a16 = reinterpret_cast<uintptr_t>(buf->tq) | reinterpret_cast<uintptr_t>(buf->tk) |
                        reinterpret_cast<uintptr_t>(buf->tv) | reinterpret_cast<uintptr_t>(buf->w_vocab) |
                        reinterpret_cast<uintptr_t>(buf->k_cache) | reinterpret_cast<uintptr_t>(buf->v_cache);
  if (a16 % 16) return fail(nullptr, MDM_E_ARG, "tables and caches must be 16-byte aligned");

  mdm_ctx* ctx = new (std::nothrow) mdm_ctx();
  if (!ctx) return fail(nullptr, MDM_E_ARG, "out of host memory");
  ctx->cfg = *cfg;
  ctx->buf = *buf;
  ctx->stream = static_cast<hipStream_t>(stream);
  ctx->L = L;
  ctx->len = 0;
  ctx->q_rows = -1;
  for (int l = 0; l <= kMaxLayers; ++l) ctx->proj_nd[l] = ctx->proj_nc[l] = -1;
  Geometry& g = ctx->g;
  g.B = cfg->batch; g.H = cfg->n_heads; g.Hkv = cfg->n_kv_heads; g.D = cfg->head_dim; g.V = cfg->vocab;
  g.seq_len = cfg->seq_len; g.R = cfg->n_registers; g.slots = (int)slots_of(cfg);
  g.table_rows = cfg->vocab + 1 + cfg->n_registers; g.max_pos = cfg->seq_len + cfg->n_registers;
  g.hidden = cfg->n_heads * cfg->head_dim; g.fp32 = cfg->precision == MDM_FP32;

  // RoPE table: theta_i = base^(-2i/d), angle = pos * theta_i, cos/sin in double, rounded to fp32.
  const int half = g.D / 2;
  std::vector<float> cs((size_t)g.max_pos * half), sn((size_t)g.max_pos * half);
  std::vector<double> theta(half);
  for (int i = 0; i < half; ++i) theta[i] = std::pow(cfg->rope_theta, -2.0 * i / g.D);
  for (int p = 0; p < g.max_pos; ++p)
    for (int i = 0; i < half; ++i) {
      const double ang = (double)p * theta[i];
      cs[(size_t)p * half + i] = (float)std::cos(ang);
      sn[(size_t)p * half + i] = (float)std::sin(ang);
    }
  mdm_status st = hip_check(ctx, hipMemcpyAsync(ctx->ws() + L.rope_cos, cs.data(), cs.size() * sizeof(float),
                                                hipMemcpyHostToDevice, ctx->stream), "upload RoPE table");
  if (st == MDM_OK)
    st = hip_check(ctx, hipMemcpyAsync(ctx->ws() + L.rope_sin, sn.data(), sn.size() * sizeof(float),
                                       hipMemcpyHostToDevice, ctx->stream), "upload RoPE table");
  if (st == MDM_OK) st = hip_check(ctx, launch_fill_i32(err_word(ctx), 0, 64, ctx->stream), "clear error flag");
  if (st == MDM_OK) st = hip_check(ctx, launch_row_norm_max(g, buf->w_vocab, wmax_word(ctx), ctx->stream), "vocab row norms");
  if (st == MDM_OK && L.wt_on)
    st = hip_check(ctx, launch_tile_w(g, buf->w_vocab, reinterpret_cast<uint16_t*>(ctx->ws() + L.wt), ctx->stream),
                   "tiled vocabulary head");
  // The packed logits rows start at zero: rows past a step's count are read
  // by the screen (their logits are never used) and must hold finite values.
  const size_t hwords = g.fp32 ? 0 : (size_t)L.m_pad * g.hidden / 2;
  if (st == MDM_OK && hwords)
    st = hip_check(ctx, launch_fill_i32(reinterpret_cast<int32_t*>(ctx->ws() + L.hhi), 0, (int)hwords, ctx->stream),
                   "clear packed rows");
  if (st == MDM_OK && hwords && cfg->accurate_conf)
    st = hip_check(ctx, launch_fill_i32(reinterpret_cast<int32_t*>(ctx->ws() + L.hlo), 0, (int)hwords, ctx->stream),
                   "clear packed rows");
  if (st == MDM_OK) {
    // Key table: the mask token rotated at every position 0..seq_len-1, then the
    // registers at seq_len..seq_len+R-1 (their keys never change).
    Geometry gt = g;
    gt.B = 1;
    gt.slots = L.ktab_rows;
    AppendArgs ka{};
    ka.tk = buf->tk; ka.tv = buf->tv; ka.kc = ctx->ws() + L.ktab; ka.vc = nullptr;
    ka.cache_pos = nullptr; ka.cache_tok = nullptr;
    ka.rope_cos = rope_cos(ctx); ka.rope_sin = rope_sin(ctx);
    ka.tok = nullptr; ka.pos = nullptr; ka.stride = 0; ka.n_a = cfg->seq_len; ka.n_reg = cfg->n_registers;
    ka.slot0 = 0; ka.err = err_word(ctx);
    st = hip_check(ctx, launch_append(gt, ka, ctx->stream), "key table");
  }
  if (st == MDM_OK && !g.fp32)
    st = hip_check(ctx, launch_value_tables(g, buf->tv, ctx->ws() + L.mvt, ctx->ws() + L.rvt, L.r_pad, ctx->stream),
                   "value tables");
  if (st == MDM_OK && !g.fp32) {
    // Query table: the key-table recipe applied to the query table over all H heads.
    Geometry gq = g;
    gq.B = 1;
    gq.Hkv = g.H;
    gq.slots = L.ktab_rows;
    AppendArgs qa{};
    qa.tk = buf->tq; qa.tv = buf->tv; qa.kc = ctx->ws() + L.qtab; qa.vc = nullptr;
    qa.cache_pos = nullptr; qa.cache_tok = nullptr;
    qa.rope_cos = rope_cos(ctx); qa.rope_sin = rope_sin(ctx);
    qa.tok = nullptr; qa.pos = nullptr; qa.stride = 0; qa.n_a = cfg->seq_len; qa.n_reg = cfg->n_registers;
    qa.slot0 = 0; qa.err = err_word(ctx);
    st = hip_check(ctx, launch_append(gq, qa, ctx->stream), "query table");
  }

  if (st == MDM_OK) st = hip_check(ctx, hipStreamSynchronize(ctx->stream), "init synchronize");
  if (st != MDM_OK) {
    delete ctx;
    return st;
  }
  *out = ctx;
  return MDM_OK;
}

mdm_status mdm_set_stream(mdm_ctx* ctx, void* stream) {
  if (!ctx) return fail(nullptr, MDM_E_ARG, "ctx is NULL");
  ctx->stream = static_cast<hipStream_t>(stream);
  return MDM_OK;
}

mdm_status mdm_kv_append(mdm_ctx* ctx, const int32_t* tok, const int32_t* pos, int64_t stride, int32_t n) {
  if (!ctx) return fail(nullptr, MDM_E_ARG, "ctx is NULL");
  if (n < 0) return fail(ctx, MDM_E_ARG, "n must be >= 0");
  if (n == 0) return MDM_OK;
  if (!tok || !pos) return fail(ctx, MDM_E_ARG, "tok and pos must be non-NULL");
  if (stride == 0) stride = n;
  if (stride < n) return fail(ctx, MDM_E_ARG, "stride %lld < n %d", (long long)stride, n);
  if ((int64_t)ctx->len + n > ctx->cfg.seq_len)
    return fail(ctx, MDM_E_CAPACITY, "cache length %d + %d exceeds seq_len %d", ctx->len, n, ctx->cfg.seq_len);
  AppendArgs a{};
  a.tk = ctx->buf.tk; a.tv = ctx->buf.tv; a.kc = ctx->buf.k_cache; a.vc = ctx->buf.v_cache;
  a.cache_pos = ctx->buf.cache_pos; a.cache_tok = ctx->buf.cache_tok;
  a.rope_cos = rope_cos(ctx); a.rope_sin = rope_sin(ctx);
  a.tok = tok; a.pos = pos; a.stride = stride; a.n_a = n; a.n_reg = 0; a.slot0 = ctx->len;
  a.err = err_word(ctx);
  // Rows that can be the D rows of the next step also get their queries.
  const bool with_q = !ctx->g.fp32 && n <= ctx->cfg.max_decode;
  if (with_q) {
    a.tq = ctx->buf.tq;
    a.qout = ctx->ws() + ctx->L.qbuf;
    a.q_rows = ctx->cfg.max_decode;
  }
  mdm_status st = hip_check(ctx, launch_append(ctx->g, a, ctx->stream), "kv_append launch");
  if (st == MDM_OK) {
    ctx->len += n;
    ctx->q_rows = with_q ? n : -1;
  }
  return st;
}

namespace {

// Launch arguments of a step attention (validated by the caller).
AttnArgs step_attn_args(mdm_ctx* ctx, const int32_t* d_tok, const int32_t* d_pos, int64_t d_stride,
                        int32_t n_new_cached, const int32_t* c_pos, int64_t c_stride, int32_t n_decode, float* out) {
  AttnArgs a{};
  a.tq = ctx->buf.tq; a.tv = ctx->buf.tv;
  a.ktab = ctx->ws() + ctx->L.ktab; a.ktab_rows = ctx->L.ktab_rows;
  if (!ctx->g.fp32) {
    a.qtab = ctx->ws() + ctx->L.qtab; a.qtab_rows = ctx->L.ktab_rows;
    if (n_new_cached > 0 && ctx->q_rows == n_new_cached) {
      a.qbuf = ctx->ws() + ctx->L.qbuf;
      a.qbuf_rows = ctx->cfg.max_decode;
    }
    a.mvt = ctx->ws() + ctx->L.mvt; a.rvt = ctx->ws() + ctx->L.rvt; a.r_pad = ctx->L.r_pad;
    a.part_o = reinterpret_cast<float*>(ctx->ws() + ctx->L.apart_o);
    a.part_ml = reinterpret_cast<float*>(ctx->ws() + ctx->L.apart_ml);
  }
  a.kc = ctx->buf.k_cache; a.vc = ctx->buf.v_cache;
  a.rope_cos = rope_cos(ctx); a.rope_sin = rope_sin(ctx);
  a.d_tok = d_tok; a.d_pos = d_pos; a.d_stride = d_stride; a.c_pos = c_pos; a.c_stride = c_stride;
  a.out = out; a.err = err_word(ctx);
  a.n_d = n_new_cached; a.n_c = n_decode; a.n_r = ctx->cfg.n_registers; a.S = ctx->len;
  return a;
}

// Launch arguments of the subset logits (validated by the caller).
VocabArgs logits_args(mdm_ctx* ctx, const float* h, int64_t h_batch_stride, int32_t n_decode, float* conf,
                      int32_t* token, float* logits_or_null) {
  VocabArgs a{};
  a.w = ctx->buf.w_vocab; a.h = h; a.h_stride = h_batch_stride; a.n_c = n_decode;
  a.hhi = reinterpret_cast<uint16_t*>(ctx->ws() + ctx->L.hhi);
  a.hlo = (ctx->cfg.precision == MDM_BF16 && ctx->cfg.accurate_conf)
              ? reinterpret_cast<uint16_t*>(ctx->ws() + ctx->L.hlo) : nullptr;
  a.partials = reinterpret_cast<float*>(ctx->ws() + ctx->L.partials);
  a.logits = logits_or_null; a.conf = conf; a.token = token; a.m_pad = ctx->L.m_pad;
  a.zpart = reinterpret_cast<float*>(ctx->ws() + ctx->L.zpart); a.zpart_bytes = (int64_t)ctx->L.zpart_bytes;
  a.v_pad = ctx->L.v_pad;
  if (ctx->L.wt_on) a.wt = reinterpret_cast<const uint16_t*>(ctx->ws() + ctx->L.wt);
  a.wmax = wmax_word(ctx);
  a.stats = decision_stats(ctx);
  a.trace = ctx->trace;
  return a;
}

}  // namespace

mdm_status mdm_step_attention(mdm_ctx* ctx, const int32_t* d_tok, const int32_t* d_pos, int64_t d_stride,
                              int32_t n_new_cached, const int32_t* c_pos, int64_t c_stride, int32_t n_decode,
                              float* out) {
  if (!ctx) return fail(nullptr, MDM_E_ARG, "ctx is NULL");
  if (!out) return fail(ctx, MDM_E_ARG, "out is NULL");
  if (n_new_cached < 0 || n_decode < 0) return fail(ctx, MDM_E_ARG, "row counts must be >= 0");
  if (n_new_cached > ctx->len)
    return fail(ctx, MDM_E_ARG, "n_new_cached %d exceeds the cache length %d", n_new_cached, ctx->len);
  if (n_decode > ctx->cfg.max_decode)
    return fail(ctx, MDM_E_ARG, "n_decode %d exceeds max_decode %d", n_decode, ctx->cfg.max_decode);
  if (n_new_cached > 0 && (!d_tok || !d_pos)) return fail(ctx, MDM_E_ARG, "d_tok/d_pos are NULL");
  if (n_decode > 0 && !c_pos) return fail(ctx, MDM_E_ARG, "c_pos is NULL");
  if (d_stride == 0) d_stride = n_new_cached;
  if (c_stride == 0) c_stride = n_decode;
  if (d_stride < n_new_cached || c_stride < n_decode) return fail(ctx, MDM_E_ARG, "stride smaller than row count");
  if ((int64_t)ctx->len + n_decode > ctx->cfg.seq_len)
    return fail(ctx, MDM_E_CAPACITY, "cache length %d + n_decode %d exceeds seq_len %d", ctx->len, n_decode,
                ctx->cfg.seq_len);
  if (n_new_cached + n_decode + ctx->cfg.n_registers == 0) return MDM_OK;
  const AttnArgs a = step_attn_args(ctx, d_tok, d_pos, d_stride, n_new_cached, c_pos, c_stride, n_decode, out);
  return hip_check(ctx, launch_attention(ctx->g, a, ctx->stream), "attention launch");
}

mdm_status mdm_subset_logits_confidence(mdm_ctx* ctx, const float* h, int64_t h_batch_stride, int32_t n_decode,
                                        float* conf, int32_t* token, float* logits_or_null) {
  if (!ctx) return fail(nullptr, MDM_E_ARG, "ctx is NULL");
  if (n_decode < 0 || n_decode > ctx->cfg.max_decode)
    return fail(ctx, MDM_E_ARG, "n_decode %d outside [0, max_decode %d]", n_decode, ctx->cfg.max_decode);
  if (n_decode == 0) return MDM_OK;
  if (!h || !conf || !token) return fail(ctx, MDM_E_ARG, "h, conf and token must be non-NULL");
  const int hidden = ctx->g.hidden;
  if (h_batch_stride == 0) h_batch_stride = (int64_t)n_decode * hidden;
  if (h_batch_stride < (int64_t)n_decode * hidden) return fail(ctx, MDM_E_ARG, "h_batch_stride too small");
  if (h_batch_stride % 4 || reinterpret_cast<uintptr_t>(h) % 16)
    return fail(ctx, MDM_E_ARG, "h must be 16-byte aligned with a stride that is a multiple of 4");
  const VocabArgs a = logits_args(ctx, h, h_batch_stride, n_decode, conf, token, logits_or_null);
  return hip_check(ctx, launch_vocab(ctx->g, a, ctx->stream), "vocab launch");
}

mdm_status mdm_order_step(mdm_ctx* ctx, int32_t n_new_cached, const int32_t* c_pos, int64_t c_stride,
                          int32_t n_decode, int32_t commit, float* out, float* conf, int32_t* token,
                          int32_t* seq_tokens, float* logits_or_null) {
  if (!ctx) return fail(nullptr, MDM_E_ARG, "ctx is NULL");
  if (ctx->g.fp32) return fail(ctx, MDM_E_UNSUPPORTED, "the fused order step needs the bf16 precision");
  if (ctx->has_upper) return fail(ctx, MDM_E_UNSUPPORTED, "the fused order step runs one attention layer");
  if (!out) return fail(ctx, MDM_E_ARG, "out is NULL");
  if (reinterpret_cast<uintptr_t>(out) % 16) return fail(ctx, MDM_E_ARG, "out must be 16-byte aligned");
  if (n_new_cached < 0 || n_decode < 0) return fail(ctx, MDM_E_ARG, "row counts must be >= 0");
  if (n_new_cached > ctx->len)
    return fail(ctx, MDM_E_ARG, "n_new_cached %d exceeds the cache length %d", n_new_cached, ctx->len);
  if (n_new_cached > 0 && ctx->q_rows != n_new_cached)
    return fail(ctx, MDM_E_ARG, "n_new_cached %d is not the row count of the preceding commit (%d)", n_new_cached,
                ctx->q_rows);
  if (n_decode > ctx->cfg.max_decode)
    return fail(ctx, MDM_E_ARG, "n_decode %d exceeds max_decode %d", n_decode, ctx->cfg.max_decode);
  if (n_decode > 0 && (!c_pos || !conf || !token)) return fail(ctx, MDM_E_ARG, "c_pos, conf and token must be non-NULL");
  if (c_stride == 0) c_stride = n_decode;
  if (c_stride < n_decode) return fail(ctx, MDM_E_ARG, "c_stride < n_decode");
  if ((int64_t)ctx->len + n_decode > ctx->cfg.seq_len)
    return fail(ctx, MDM_E_CAPACITY, "cache length %d + n_decode %d exceeds seq_len %d", ctx->len, n_decode,
                ctx->cfg.seq_len);
  const int n_r = ctx->cfg.n_registers;
  if (n_new_cached + n_decode + n_r == 0) return MDM_OK;
  AttnArgs a = step_attn_args(ctx, nullptr, nullptr, 0, n_new_cached, c_pos, c_stride, n_decode, out);
  const int hidden = ctx->g.hidden;
  VocabArgs v = logits_args(ctx, out + (int64_t)n_new_cached * hidden, (int64_t)(n_new_cached + n_decode + n_r) * hidden,
                            n_decode, conf, token, logits_or_null);
  if (n_decode > 0) {
    a.pack_hi = v.hhi;
    a.pack_lo = v.hlo;
  }
  mdm_status st = hip_check(ctx, launch_attention(ctx->g, a, ctx->stream), "attention launch");
  if (st != MDM_OK || n_decode == 0) return st;
  v.prepacked = 1;
  v.cand_pos = c_pos; v.cand_stride = c_stride; v.seq_tokens = seq_tokens; v.err = err_word(ctx);
  st = hip_check(ctx, launch_vocab(ctx->g, v, ctx->stream), "vocab launch");
  if (st == MDM_OK && commit) {
    // the decided rows enter the cache as mdm_kv_append(token, c_pos) would
    // append them: one launch over 32-row blocks
    AppendArgs ca{};
    ca.tk = ctx->buf.tk; ca.tv = ctx->buf.tv; ca.kc = ctx->buf.k_cache; ca.vc = ctx->buf.v_cache;
    ca.cache_pos = ctx->buf.cache_pos; ca.cache_tok = ctx->buf.cache_tok;
    ca.rope_cos = rope_cos(ctx); ca.rope_sin = rope_sin(ctx);
    ca.tok = token; ca.stride = n_decode; ca.pos = c_pos; ca.pos_stride = c_stride;
    ca.n_a = n_decode; ca.slot0 = ctx->len; ca.err = err_word(ctx);
    ca.tq = ctx->buf.tq; ca.qout = ctx->ws() + ctx->L.qbuf; ca.q_rows = ctx->cfg.max_decode;
    st = hip_check(ctx, launch_append(ctx->g, ca, ctx->stream), "commit launch");
  }
  if (st == MDM_OK && commit) {
    ctx->len += n_decode;
    ctx->q_rows = n_decode;
  }
  return st;
}

mdm_status mdm_unmask_select(mdm_ctx* ctx, const int32_t* cand_pos, int64_t cand_stride, const float* conf,
                             const int32_t* token, int32_t n_cand, int32_t n_select, int32_t mode, int32_t* out_tok,
                             int32_t* out_pos, int32_t* rem_pos, int32_t* seq_tokens) {
  if (!ctx) return fail(nullptr, MDM_E_ARG, "ctx is NULL");
  if (n_cand < 0 || n_cand > kMaxSelectCand) return fail(ctx, MDM_E_ARG, "n_cand outside [0, %d]", kMaxSelectCand);
  if (n_select < 0 || n_select > n_cand) return fail(ctx, MDM_E_ARG, "n_select outside [0, n_cand]");
  if (mode != MDM_SELECT_ORDER && mode != MDM_SELECT_CONFIDENCE) return fail(ctx, MDM_E_ARG, "unknown mode");
  if (mode == MDM_SELECT_ORDER && n_select != n_cand)
    return fail(ctx, MDM_E_ARG, "order mode unmasks every candidate (n_select must equal n_cand)");
  if (n_cand == 0) return MDM_OK;
  if (!cand_pos || !token || !out_tok || !out_pos) return fail(ctx, MDM_E_ARG, "a required pointer is NULL");
  if (mode == MDM_SELECT_CONFIDENCE && !conf) return fail(ctx, MDM_E_ARG, "conf is NULL");
  if (cand_stride == 0) cand_stride = n_cand;
  if (cand_stride < n_cand) return fail(ctx, MDM_E_ARG, "cand_stride < n_cand");
  SelectArgs a{};
  a.cand_pos = cand_pos; a.cand_stride = cand_stride; a.conf = conf; a.token = token;
  a.n_cand = n_cand; a.n_select = n_select; a.by_conf = mode == MDM_SELECT_CONFIDENCE;
  a.out_tok = out_tok; a.out_pos = out_pos; a.rem_pos = rem_pos; a.seq_tokens = seq_tokens;
  a.err = err_word(ctx);
  return hip_check(ctx, launch_select(ctx->g, a, ctx->stream), "select launch");
}

mdm_status mdm_sparse_step_reset(mdm_ctx* ctx) {
  if (!ctx) return fail(nullptr, MDM_E_ARG, "ctx is NULL");
  ctx->len = 0;
  ctx->q_rows = -1;
  for (int l = 0; l <= kMaxLayers; ++l) {
    ctx->len_up[l] = 0;
    ctx->proj_nd[l] = ctx->proj_nc[l] = -1;
  }
  return MDM_OK;
}

size_t mdm_upper_workspace_bytes(const mdm_config* cfg) {
  if (!config_ok(cfg, nullptr) || cfg->precision != MDM_BF16) return 0;
  return upper_layout_of(cfg).total;
}

mdm_status mdm_attach_upper_layers(mdm_ctx* ctx, const mdm_upper_layers* up) {
  if (!ctx) return fail(nullptr, MDM_E_ARG, "ctx is NULL");
  if (!up) return fail(ctx, MDM_E_ARG, "upper layers are NULL");
  if (ctx->cfg.precision != MDM_BF16) return fail(ctx, MDM_E_UNSUPPORTED, "upper layers need the bf16 precision");
  if (up->n_layers < 2 || up->n_layers > kMaxLayers)
    return fail(ctx, MDM_E_ARG, "n_layers %d out of range 2..%d", up->n_layers, kMaxLayers);
  if (!up->w_upper || !up->k_cache_upper || !up->v_cache_upper || !up->workspace)
    return fail(ctx, MDM_E_ARG, "a required upper-layer pointer is NULL");
  if (((uintptr_t)up->w_upper | (uintptr_t)up->k_cache_upper | (uintptr_t)up->v_cache_upper) % 16)
    return fail(ctx, MDM_E_ARG, "upper-layer weights and caches must be 16-byte aligned");
  if ((uintptr_t)up->workspace % kAlign) return fail(ctx, MDM_E_ARG, "upper workspace must be 256-byte aligned");
  const UpperLayout U = upper_layout_of(&ctx->cfg);
  if (up->workspace_bytes < U.total)
    return fail(ctx, MDM_E_SHAPE, "upper workspace has %zu bytes, needs %zu", up->workspace_bytes, U.total);
  ctx->up = *up;
  ctx->U = U;
  ctx->has_upper = true;
  for (int l = 0; l <= kMaxLayers; ++l) {
    ctx->len_up[l] = 0;
    ctx->proj_nd[l] = ctx->proj_nc[l] = -1;
  }
  return MDM_OK;
}

namespace {
size_t upper_cache_elems(const mdm_ctx* ctx) {
  return (size_t)ctx->cfg.batch * ctx->cfg.n_kv_heads * ctx->g.slots * ctx->cfg.head_dim;
}
mdm_status upper_layer_ok(mdm_ctx* ctx, int32_t layer) {
  if (!ctx->has_upper) return fail(ctx, MDM_E_ARG, "no upper layers attached");
  if (layer < 2 || layer > ctx->up.n_layers)
    return fail(ctx, MDM_E_ARG, "layer %d out of range 2..%d", layer, ctx->up.n_layers);
  return MDM_OK;
}
}  // namespace

mdm_status mdm_layer_project(mdm_ctx* ctx, int32_t layer, const float* h_prev, int64_t h_batch_stride,
                             const int32_t* d_pos, int64_t d_stride, int32_t n_new_cached, const int32_t* c_pos,
                             int64_t c_stride, int32_t n_decode) {
  if (!ctx) return fail(nullptr, MDM_E_ARG, "ctx is NULL");
  mdm_status st = upper_layer_ok(ctx, layer);
  if (st != MDM_OK) return st;
  if (!h_prev) return fail(ctx, MDM_E_ARG, "h_prev is NULL");
  if (n_new_cached < 0 || n_decode < 0) return fail(ctx, MDM_E_ARG, "row counts must be >= 0");
  if (n_new_cached > 0 && !d_pos) return fail(ctx, MDM_E_ARG, "d_pos is NULL");
  if (n_decode > 0 && !c_pos) return fail(ctx, MDM_E_ARG, "c_pos is NULL");
  if (n_decode > ctx->cfg.max_decode)
    return fail(ctx, MDM_E_ARG, "n_decode %d exceeds max_decode %d", n_decode, ctx->cfg.max_decode);
  if (d_stride == 0) d_stride = n_new_cached;
  if (c_stride == 0) c_stride = n_decode;
  if (d_stride < n_new_cached || c_stride < n_decode) return fail(ctx, MDM_E_ARG, "stride smaller than row count");
  const int n_q = n_new_cached + n_decode + ctx->cfg.n_registers;
  const int hidden = ctx->g.hidden;
  if (h_batch_stride == 0) h_batch_stride = (int64_t)n_q * hidden;
  if (h_batch_stride < (int64_t)n_q * hidden) return fail(ctx, MDM_E_ARG, "h_batch_stride smaller than the rows");
  if ((uintptr_t)h_prev % 16 || h_batch_stride % 4) return fail(ctx, MDM_E_ARG, "h rows must be 16-byte aligned");
  if (n_q > ctx->U.q_rows) return fail(ctx, MDM_E_CAPACITY, "%d rows exceed seq_len + R", n_q);
  if ((int64_t)ctx->len_up[layer] + n_new_cached > ctx->cfg.seq_len)
    return fail(ctx, MDM_E_CAPACITY, "layer %d cache length %d + %d exceeds seq_len %d", layer, ctx->len_up[layer],
                n_new_cached, ctx->cfg.seq_len);
  if (n_q == 0) return MDM_OK;
  const UpperLayout& U = ctx->U;
  const size_t w_elems = (size_t)(ctx->cfg.n_heads + 2 * ctx->cfg.n_kv_heads) * ctx->cfg.head_dim * hidden;
  ProjArgs p{};
  p.w = static_cast<const uint16_t*>(ctx->up.w_upper) + (size_t)(layer - 2) * w_elems;
  p.h = h_prev;
  p.h_stride = h_batch_stride;
  p.n_d = n_new_cached; p.n_c = n_decode; p.n_q = n_q;
  p.d_pos = d_pos; p.d_stride = d_stride; p.c_pos = c_pos; p.c_stride = c_stride;
  p.hhi = reinterpret_cast<uint16_t*>(ctx->uws() + U.hhi);
  p.hlo = reinterpret_cast<uint16_t*>(ctx->uws() + U.hlo);
  p.z = reinterpret_cast<float*>(ctx->uws() + U.z);
  p.n_pad = U.n_pad;
  p.rope_cos = rope_cos(ctx); p.rope_sin = rope_sin(ctx);
  p.qbuf = ctx->uws() + U.qbuf; p.qbuf_rows = U.q_rows;
  p.kc = static_cast<uint16_t*>(ctx->up.k_cache_upper) + (size_t)(layer - 2) * upper_cache_elems(ctx);
  p.vc = static_cast<uint16_t*>(ctx->up.v_cache_upper) + (size_t)(layer - 2) * upper_cache_elems(ctx);
  p.slot0 = ctx->len_up[layer];
  p.tk = ctx->uws() + U.tk; p.tvt = ctx->uws() + U.tvt; p.t_pad = U.t_pad;
  p.err = err_word(ctx);
  st = hip_check(ctx, launch_project(ctx->g, p, ctx->stream), "projection launch");
  if (st != MDM_OK) return st;
  ctx->len_up[layer] += n_new_cached;
  ctx->proj_nd[layer] = n_new_cached;
  ctx->proj_nc[layer] = n_decode;
  return MDM_OK;
}

mdm_status mdm_layer_attention(mdm_ctx* ctx, int32_t layer, int32_t n_new_cached, int32_t n_decode, float* out) {
  if (!ctx) return fail(nullptr, MDM_E_ARG, "ctx is NULL");
  mdm_status st = upper_layer_ok(ctx, layer);
  if (st != MDM_OK) return st;
  if (!out) return fail(ctx, MDM_E_ARG, "out is NULL");
  if (ctx->proj_nd[layer] != n_new_cached || ctx->proj_nc[layer] != n_decode)
    return fail(ctx, MDM_E_ARG, "layer %d: the latest projection had %d new and %d decoded rows, not %d and %d",
                layer, ctx->proj_nd[layer], ctx->proj_nc[layer], n_new_cached, n_decode);
  const int n_r = ctx->cfg.n_registers;
  if (n_new_cached + n_decode + n_r == 0) return MDM_OK;
  AttnArgs a{};
  a.tq = ctx->buf.tq; a.tv = ctx->buf.tv;
  a.ktab = ctx->ws() + ctx->L.ktab; a.ktab_rows = ctx->L.ktab_rows;
  a.qtab = ctx->ws() + ctx->L.qtab; a.qtab_rows = ctx->L.ktab_rows;
  a.qbuf = ctx->uws() + ctx->U.qbuf; a.qbuf_rows = ctx->U.q_rows;
  a.mvt = ctx->ws() + ctx->L.mvt; a.rvt = ctx->ws() + ctx->L.rvt; a.r_pad = ctx->U.t_pad;
  a.part_o = reinterpret_cast<float*>(ctx->ws() + ctx->L.apart_o);
  a.part_ml = reinterpret_cast<float*>(ctx->ws() + ctx->L.apart_ml);
  a.kc = static_cast<uint16_t*>(ctx->up.k_cache_upper) + (size_t)(layer - 2) * upper_cache_elems(ctx);
  a.vc = static_cast<uint16_t*>(ctx->up.v_cache_upper) + (size_t)(layer - 2) * upper_cache_elems(ctx);
  a.rope_cos = rope_cos(ctx); a.rope_sin = rope_sin(ctx);
  a.out = out; a.err = err_word(ctx);
  // C and R rows see the same keys: one transient segment of n_decode + R keys
  a.n_d = n_new_cached; a.n_c = 0; a.n_r = n_decode + n_r; a.S = ctx->len_up[layer];
  a.tk = ctx->uws() + ctx->U.tk; a.tvt = ctx->uws() + ctx->U.tvt; a.t_pad = ctx->U.t_pad;
  return hip_check(ctx, launch_attention(ctx->g, a, ctx->stream), "layer attention launch");
}

int32_t mdm_cache_len(const mdm_ctx* ctx) { return ctx ? ctx->len : -1; }

mdm_status mdm_cache_rewind(mdm_ctx* ctx, int32_t new_len) {
  if (!ctx) return fail(nullptr, MDM_E_ARG, "ctx is NULL");
  if (ctx->has_upper) return fail(ctx, MDM_E_UNSUPPORTED, "rewind with upper layers attached");
  if (new_len < 0 || new_len > ctx->len)
    return fail(ctx, MDM_E_ARG, "new length %d outside [0, cache length %d]", new_len, ctx->len);
  if (new_len != ctx->len) ctx->q_rows = -1;
  ctx->len = new_len;
  return MDM_OK;
}

mdm_status mdm_set_decision_trace(mdm_ctx* ctx, float* trace) {
  if (!ctx) return fail(nullptr, MDM_E_ARG, "ctx is NULL");
  if (reinterpret_cast<uintptr_t>(trace) % 16) return fail(ctx, MDM_E_ARG, "trace must be 16-byte aligned");
  ctx->trace = trace;
  return MDM_OK;
}

mdm_status mdm_decision_counts(mdm_ctx* ctx, int64_t* out) {
  if (!ctx) return fail(nullptr, MDM_E_ARG, "ctx is NULL");
  if (!out) return fail(ctx, MDM_E_ARG, "out is NULL");
  unsigned c[3] = {0, 0, 0};
  mdm_status st = hip_check(ctx, hipMemcpyAsync(c, decision_stats(ctx), sizeof c, hipMemcpyDeviceToHost, ctx->stream),
                            "read decision counters");
  if (st == MDM_OK) st = hip_check(ctx, hipStreamSynchronize(ctx->stream), "synchronize");
  if (st == MDM_OK)
    st = hip_check(ctx, launch_fill_i32(reinterpret_cast<int32_t*>(decision_stats(ctx)), 0, 3, ctx->stream),
                   "clear decision counters");
  if (st != MDM_OK) return st;
  for (int i = 0; i < 3; ++i) out[i] = c[i];
  return MDM_OK;
}

mdm_status mdm_device_status(mdm_ctx* ctx) {
  if (!ctx) return fail(nullptr, MDM_E_ARG, "ctx is NULL");
  int flag = 0;
  mdm_status st = hip_check(ctx, hipMemcpyAsync(&flag, err_word(ctx), sizeof(int), hipMemcpyDeviceToHost, ctx->stream),
                            "read error flag");
  if (st == MDM_OK) st = hip_check(ctx, hipStreamSynchronize(ctx->stream), "synchronize");
  if (st != MDM_OK) return st;
  if (flag) {
    st = hip_check(ctx, launch_fill_i32(err_word(ctx), 0, 1, ctx->stream), "clear error flag");
    if (st != MDM_OK) return st;
    return fail(ctx, MDM_E_DEVICE, "kernels met an out-of-range %s%s", (flag & kErrTok) ? "token id " : "",
                (flag & kErrPos) ? "position" : "");
  }
  return MDM_OK;
}

namespace {
constexpr int kBlockAttnHeadDim = 128;
bool block_shape_ok(const mdm_block_attn_shape* s) {
  return s && s->batch > 0 && s->n_rows > 0 && s->n_heads > 0 && s->n_kv_heads > 0 &&
         s->n_heads % s->n_kv_heads == 0;
}
size_t block_ws_bytes(const mdm_block_attn_shape* s) {
  return (size_t)s->batch * ((s->n_rows + kKeyTile - 1) / kKeyTile) * 2 * sizeof(int32_t);
}
}  // namespace

size_t mdm_block_attention_workspace_bytes(const mdm_block_attn_shape* shape) {
  return block_shape_ok(shape) ? block_ws_bytes(shape) : 0;
}

namespace {
// Shape and pointer checks shared by both block-attention entry points.
mdm_status block_attention_check(const mdm_block_attn_shape* s, const uint16_t* q, const uint16_t* k,
                                 const uint16_t* v, const int32_t* blocks, const int32_t* n_clean_blocks,
                                 const float* out) {
  if (!block_shape_ok(s))
    return fail(nullptr, MDM_E_ARG, "block attention: sizes must be positive and n_heads a multiple of n_kv_heads");
  if (s->head_dim != kBlockAttnHeadDim)
    return fail(nullptr, MDM_E_UNSUPPORTED, "block attention: head_dim %d (only 128)", s->head_dim);
  if (s->n_rows > kBlockAttnMaxTiles * kKeyTile)
    return fail(nullptr, MDM_E_UNSUPPORTED, "block attention: %d rows (at most %d)", s->n_rows,
                kBlockAttnMaxTiles * kKeyTile);
  if (!q || !k || !v || !blocks || !n_clean_blocks || !out)
    return fail(nullptr, MDM_E_ARG, "block attention: a required pointer is NULL");
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out) % 16)
    return fail(nullptr, MDM_E_ARG, "block attention: q, k, v and out must be 16-byte aligned");
  return MDM_OK;
}
}  // namespace

mdm_status mdm_block_attention(const mdm_block_attn_shape* s, const uint16_t* q, const uint16_t* k,
                               const uint16_t* v, const int32_t* blocks, const int32_t* n_clean_blocks,
                               float* out, void* workspace, size_t workspace_bytes, void* stream) {
  mdm_status st = block_attention_check(s, q, k, v, blocks, n_clean_blocks, out);
  if (st != MDM_OK) return st;
  if (!workspace) return fail(nullptr, MDM_E_ARG, "block attention: a required pointer is NULL");
  if ((uintptr_t)workspace % 4) return fail(nullptr, MDM_E_ARG, "block attention: workspace must be 4-byte aligned");
  if (workspace_bytes < block_ws_bytes(s))
    return fail(nullptr, MDM_E_SHAPE, "block attention: workspace has %zu bytes, needs %zu", workspace_bytes,
                block_ws_bytes(s));
  BlockAttnArgs a{};
  a.q = q; a.k = k; a.v = v; a.blk = blocks; a.n_clean = n_clean_blocks; a.out = out;
  a.ranges = static_cast<int32_t*>(workspace);
  a.B = s->batch; a.n = s->n_rows; a.H = s->n_heads; a.Hkv = s->n_kv_heads;
  return hip_check(nullptr, launch_block_attention(a, static_cast<hipStream_t>(stream)), "block attention launch");
}

mdm_status mdm_block_attention_static(const mdm_block_attn_shape* s, const uint16_t* q, const uint16_t* k,
                                      const uint16_t* v, const int32_t* blocks, const int32_t* n_clean_blocks,
                                      float* out, void* stream) {
  mdm_status st = block_attention_check(s, q, k, v, blocks, n_clean_blocks, out);
  if (st != MDM_OK) return st;
  int32_t* ranges = nullptr;
  size_t cap = 0;
  st = hip_check(nullptr, block_attention_static_scratch(&ranges, &cap), "block attention: static range array");
  if (st != MDM_OK) return st;
  const size_t need = block_ws_bytes(s) / sizeof(int32_t);
  if (need > cap)
    return fail(nullptr, MDM_E_UNSUPPORTED,
                "block attention (static): batch * ceil(n_rows / 64) = %zu tile ranges, at most %zu", need / 2,
                cap / 2);
  BlockAttnArgs a{};
  a.q = q; a.k = k; a.v = v; a.blk = blocks; a.n_clean = n_clean_blocks; a.out = out;
  a.ranges = ranges;
  a.B = s->batch; a.n = s->n_rows; a.H = s->n_heads; a.Hkv = s->n_kv_heads;
  return hip_check(nullptr, launch_block_attention(a, static_cast<hipStream_t>(stream)), "block attention launch");
}

void mdm_sparse_step_destroy(mdm_ctx* ctx) { delete ctx; }

const char* mdm_last_error(const mdm_ctx* ctx) { return ctx ? ctx->err.c_str() : g_last_error.c_str(); }

const char* mdm_status_string(int32_t s) {
  switch (s) {
    case MDM_OK: return "MDM_OK";
    case MDM_E_ARG: return "MDM_E_ARG";
    case MDM_E_SHAPE: return "MDM_E_SHAPE";
    case MDM_E_CAPACITY: return "MDM_E_CAPACITY";
    case MDM_E_HIP: return "MDM_E_HIP";
    case MDM_E_UNSUPPORTED: return "MDM_E_UNSUPPORTED";
    case MDM_E_DEVICE: return "MDM_E_DEVICE";
    default: return "MDM_E_UNKNOWN";
  }
}

}  // extern "C"
