// C ABI of the MoT world-action-model forward pass (declared in wam.h and
// wam_ops.h): packed-weight layout, workspace layout, argument validation,
// and the two schedules of the same kernels:
//   sequential -- video expert, then the S action passes, on one stream;
//   wavefront  -- video expert on s_video, action expert on s_action; the
//                 video stream records event e_i right after block i's merged
//                 q|k|v projection has written (K^v_i, V^v_i) into the cache,
//                 and the action stream waits on e_i only immediately before
//                 its block-i attention (RealtimeWAM digest, "Core method" and
//                 "Method steps": record after P^v_i, wait before Attn^a_i).
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <array>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.h"
#include "wam.h"
#include "wam_ops.h"

// ============================================================================
// errors
// ============================================================================
static thread_local std::string g_err;

static int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

#define HIP_TRY(expr)                                                                         \
  do {                                                                                        \
    hipError_t _e = (expr);                                                                   \
    if (_e != hipSuccess) return fail(WAM_ERR_HIP, std::string(#expr) + ": " + hipGetErrorString(_e)); \
  } while (0)

extern "C" const char* wam_last_error(void) { return g_err.c_str(); }

// ============================================================================
// configuration and packed weight layout
// ============================================================================
static int check_config(const wam_config* c) {
  if (!c) return fail(WAM_ERR_NULL, "config is NULL");
  if (c->dtype != WAM_F32 && c->dtype != WAM_BF16) return fail(WAM_ERR_DTYPE, "dtype must be WAM_F32 or WAM_BF16");
  auto bad = [](const char* what) { return fail(WAM_ERR_SHAPE, std::string("invalid config: ") + what); };
  if (c->n_blocks < 1 || c->n_blocks > 1024) return bad("n_blocks");
  for (int d : {c->d_video, c->d_action})
    if (d < 64 || d > 8192 || d % 64) return bad("d_video/d_action must be multiples of 64 in [64, 8192]");
  if (c->head_dim != 32 && c->head_dim != 64 && c->head_dim != 128) return bad("head_dim must be 32, 64 or 128");
  if (c->dtype == WAM_BF16 && c->head_dim == 32) return bad("bf16 models need head_dim 64 or 128");
  if (c->n_heads < 1 || (c->n_heads * c->head_dim) % 64 || c->n_heads * c->head_dim > 16384) return bad("n_heads");
  if (c->mlp_ratio < 1 || c->mlp_ratio > 16) return bad("mlp_ratio");
  if (c->t_freq_dim < 8 || c->t_freq_dim > 1024 || c->t_freq_dim % 8) return bad("t_freq_dim must be a multiple of 8 in [8, 1024]");
  if (c->action_dim < 1 || c->action_dim > 64) return bad("action_dim must be in [1, 64]");
  if (c->max_batch < 1 || c->max_video_tokens < 0 || c->max_action_tokens < 1) return bad("max sizes");
  if (c->max_steps < 1 || c->max_steps > WAM_MAX_T) return bad("max_steps must be in [1, 64]");
  if ((long long)c->max_batch * c->max_video_tokens > (1LL << 26) ||
      (long long)c->max_batch * c->max_action_tokens > (1LL << 20))
    return bad("max token counts too large");
  if (!(c->ln_eps > 0.0f) || !isfinite(c->ln_eps)) return bad("ln_eps must be > 0");
  if (c->qk_norm != 0 && c->qk_norm != 1) return bad("qk_norm must be 0 or 1");
  if ((c->rope_height == 0) != (c->rope_width == 0) || c->rope_height < 0 || c->rope_width < 0 ||
      c->rope_height > 4096 || c->rope_width > 4096)
    return bad("rope_height and rope_width must both be 0 or both in [1, 4096]");
  return WAM_OK;
}

struct TensorDesc {
  std::string name;
  int rows, cols;
  size_t off;
};

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Tensor offsets.  Each expert: its t-MLP, then every block's adaLN matrix
// back to back (the action expert's final-layer adaLN right after them),
// then the adaLN biases likewise, then the per-block projection/MLP weights.
static std::vector<TensorDesc> build_layout(const wam_config& c, size_t* total) {
  const size_t es = c.dtype == WAM_F32 ? 4 : 2;
  const int D = c.n_heads * c.head_dim;
  std::vector<TensorDesc> t;
  size_t off = 0;
  auto add = [&](const std::string& n, int r, int cols) {
    off = align256(off);
    t.push_back({n, r, cols, off});
    off += (size_t)r * cols * es;
  };
  for (int ex = 0; ex < 2; ++ex) {
    const std::string p = ex == 0 ? "v." : "a.";
    const int d = ex == 0 ? c.d_video : c.d_action;
    if (ex == 1) {
      add("a.in.w", d, c.action_dim);
      add("a.in.b", 1, d);
    }
    add(p + "t1.w", d, c.t_freq_dim);
    add(p + "t1.b", 1, d);
    add(p + "t2.w", d, d);
    add(p + "t2.b", 1, d);
    off = align256(off);
    for (int i = 0; i < c.n_blocks; ++i) {
      t.push_back({p + std::to_string(i) + ".ada.w", 6 * d, d, off});
      off += (size_t)6 * d * d * es;
    }
    if (ex == 1) {
      t.push_back({"a.fada.w", 2 * d, d, off});
      off += (size_t)2 * d * d * es;
    }
    off = align256(off);
    for (int i = 0; i < c.n_blocks; ++i) {
      t.push_back({p + std::to_string(i) + ".ada.b", 1, 6 * d, off});
      off += (size_t)6 * d * es;
    }
    if (ex == 1) {
      t.push_back({"a.fada.b", 1, 2 * d, off});
      off += (size_t)2 * d * es;
    }
    for (int i = 0; i < c.n_blocks; ++i) {
      const std::string b = p + std::to_string(i) + ".";
      add(b + "qkv.w", 3 * D, d);
      add(b + "qkv.b", 1, 3 * D);
      add(b + "o.w", d, D);
      add(b + "o.b", 1, d);
      add(b + "fc1.w", c.mlp_ratio * d, d);
      add(b + "fc1.b", 1, c.mlp_ratio * d);
      add(b + "fc2.w", d, c.mlp_ratio * d);
      add(b + "fc2.b", 1, d);
    }
    if (ex == 1) {
      add("a.out.w", c.action_dim, d);
      add("a.out.b", 1, c.action_dim);
    }
  }
  if (c.qk_norm)
    for (int ex = 0; ex < 2; ++ex)
      for (int i = 0; i < c.n_blocks; ++i) {
        const std::string b = (ex == 0 ? "v." : "a.") + std::to_string(i) + ".";
        add(b + "qn.g", 1, D);
        add(b + "kn.g", 1, D);
      }
  *total = align256(off);
  return t;
}

extern "C" int wam_config_check(const wam_config* cfg) { return check_config(cfg); }

extern "C" int wam_weights_tensor_count(const wam_config* cfg) {
  if (check_config(cfg) != WAM_OK) return 0;
  size_t total;
  return (int)build_layout(*cfg, &total).size();
}

extern "C" size_t wam_weights_bytes(const wam_config* cfg) {
  if (check_config(cfg) != WAM_OK) return 0;
  size_t total;
  build_layout(*cfg, &total);
  return total;
}

extern "C" int wam_weights_tensor_info(const wam_config* cfg, int index, wam_tensor_info* out) {
  int rc = check_config(cfg);
  if (rc != WAM_OK) return rc;
  if (!out) return fail(WAM_ERR_NULL, "out is NULL");
  size_t total;
  std::vector<TensorDesc> t = build_layout(*cfg, &total);
  if (index < 0 || index >= (int)t.size()) return fail(WAM_ERR_SHAPE, "tensor index out of range");
  memset(out, 0, sizeof(*out));
  snprintf(out->name, sizeof(out->name), "%s", t[index].name.c_str());
  out->rows = t[index].rows;
  out->cols = t[index].cols;
  out->offset_bytes = t[index].off;
  return WAM_OK;
}

// ============================================================================
// fixed scratch of wam_action_step_noalloc: one array per GPU, allocated with
// the code object and held until the process ends.  In host code `scratch`
// names a host-side stand-in, never the device memory: its address on a
// device is taken once per device, at model creation (that device current),
// and only that address is handed to kernels.
// ============================================================================
static __device__ __align__(256) unsigned char scratch[WAM_NOALLOC_SCRATCH_BYTES];
static std::mutex g_scratch_mu;
static std::map<int, void*> g_scratch_dev;  // device ordinal -> address of its scratch

static int scratch_setup(int device) {  // `device` is current
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (g_scratch_dev.count(device)) return WAM_OK;
  void* ptr = nullptr;
  hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !ptr)
    return fail(WAM_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
  g_scratch_dev[device] = ptr;
  return WAM_OK;
}

static void* scratch_of(int device) {
  std::lock_guard<std::mutex> g(g_scratch_mu);
  auto it = g_scratch_dev.find(device);
  return it == g_scratch_dev.end() ? nullptr : it->second;
}

// ============================================================================
// model
// ============================================================================
struct BlockW {
  const void *qkv_w, *qkv_b, *o_w, *o_b, *fc1_w, *fc1_b, *fc2_w, *fc2_b;
  const void *qn_g, *kn_g;  // QK-RMSNorm gains (NULL without the variant)
};
struct ExpertW {
  const void *t1_w, *t1_b, *t2_w, *t2_b, *ada_w, *ada_b;
  std::vector<BlockW> blk;
};

struct wam_model {
  wam_config cfg;
  const uint8_t* w;
  ExpertW vid, act;
  const void *in_w, *in_b, *out_w, *out_b;
  std::vector<hipEvent_t> ev_block;
  hipEvent_t ev_fork = nullptr, ev_join = nullptr;
  int device = 0;
  // debug hooks (environment, read when the model is created): a wait of
  // this many microseconds at the start of every video block / right after
  // every action block's wait for its video block; results never depend on them
  uint32_t delay_video_us = 0, delay_action_us = 0;
};

// WAM_DEBUG_VIDEO_DELAY_US / WAM_DEBUG_ACTION_DELAY_US: a decimal count of
// microseconds (capped at kMaxDebugDelayUs); anything else means no delay.
static uint32_t env_delay_us(const char* name) {
  const char* v = getenv(name);
  if (!v || !*v) return 0;
  char* end = nullptr;
  const unsigned long x = strtoul(v, &end, 10);
  return *end == 0 ? (uint32_t)std::min<unsigned long>(x, kMaxDebugDelayUs) : 0u;
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }
// A prefetch range for the attention kernel: whole 4-byte words, under 4 GB
// (its offsets are 32-bit; a larger range is only touched in its first 4 GB).
static uint32_t prefetch_bytes(size_t n) { return (uint32_t)std::min<size_t>(n, 0xFFFFF000u) & ~3u; }

extern "C" int wam_model_create(const wam_config* cfg, const void* weights_dev, wam_model** out) {
  int rc = check_config(cfg);
  if (rc != WAM_OK) return rc;
  if (!weights_dev || !out) return fail(WAM_ERR_NULL, "weights_dev and out must be non-NULL");
  if (((uintptr_t)weights_dev & 255) != 0) return fail(WAM_ERR_ALIGN, "weights_dev must be 256-byte aligned");
  size_t total;
  std::vector<TensorDesc> t = build_layout(*cfg, &total);
  wam_model* m = new wam_model();
  m->cfg = *cfg;
  m->delay_video_us = env_delay_us("WAM_DEBUG_VIDEO_DELAY_US");
  m->delay_action_us = env_delay_us("WAM_DEBUG_ACTION_DELAY_US");
  m->w = (const uint8_t*)weights_dev;
  auto find = [&](const std::string& n) -> const void* {
    for (const auto& d : t)
      if (d.name == n) return m->w + d.off;
    return nullptr;
  };
  for (int ex = 0; ex < 2; ++ex) {
    const std::string p = ex == 0 ? "v." : "a.";
    ExpertW& e = ex == 0 ? m->vid : m->act;
    e.t1_w = find(p + "t1.w");
    e.t1_b = find(p + "t1.b");
    e.t2_w = find(p + "t2.w");
    e.t2_b = find(p + "t2.b");
    e.ada_w = find(p + "0.ada.w");
    e.ada_b = find(p + "0.ada.b");
    for (int i = 0; i < cfg->n_blocks; ++i) {
      const std::string b = p + std::to_string(i) + ".";
      e.blk.push_back({find(b + "qkv.w"), find(b + "qkv.b"), find(b + "o.w"), find(b + "o.b"), find(b + "fc1.w"),
                       find(b + "fc1.b"), find(b + "fc2.w"), find(b + "fc2.b"), find(b + "qn.g"), find(b + "kn.g")});
    }
  }
  m->in_w = find("a.in.w");
  m->in_b = find("a.in.b");
  m->out_w = find("a.out.w");
  m->out_b = find("a.out.b");
  // The events only order the two streams of one device (fork, join, one per
  // video block); nothing on the host or another device inspects them, so
  // they skip the system-scope fence a default event adds when recorded.
  // Device-scope ordering between the streams' kernels is unaffected.
  const unsigned ev_flags = hipEventDisableTiming | hipEventDisableSystemFence;
  hipError_t e = hipGetDevice(&m->device);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&m->ev_fork, ev_flags);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&m->ev_join, ev_flags);
  for (int i = 0; e == hipSuccess && i < cfg->n_blocks; ++i) {
    hipEvent_t ev;
    e = hipEventCreateWithFlags(&ev, ev_flags);
    if (e == hipSuccess) m->ev_block.push_back(ev);
  }
  if (e != hipSuccess) {
    wam_model_destroy(m);
    return fail(WAM_ERR_HIP, std::string("creating events: ") + hipGetErrorString(e));
  }
  rc = scratch_setup(m->device);
  if (rc != WAM_OK) {
    std::string msg = g_err;
    wam_model_destroy(m);
    return fail(rc, msg);
  }
  *out = m;
  return WAM_OK;
}

extern "C" int wam_model_destroy(wam_model* m) {
  if (!m) return fail(WAM_ERR_NULL, "model is NULL");
  for (hipEvent_t ev : m->ev_block) (void)hipEventDestroy(ev);
  if (m->ev_fork) (void)hipEventDestroy(m->ev_fork);
  if (m->ev_join) (void)hipEventDestroy(m->ev_join);
  delete m;
  return WAM_OK;
}

// ============================================================================
// workspace
// ============================================================================
struct WsLayout {
  // video expert
  size_t v_e, v_h1, v_c, v_mod, v_x, v_h, v_q, v_o, v_g, v_part;
  // action expert
  size_t a_e, a_h1, a_c, a_mod, a_y, a_h, a_q, a_k, a_v, a_o, a_g, a_part, a_attn, a_cur;
  // teacher-anchored targets: a_t and a second Euler buffer
  size_t g_at, g_alt;
  // selective reuse: active token indices (T_v ints) and their count
  size_t r_idx, r_count;
  size_t total;
};

// Scratch (floats) of the video pass over n active rows of one sample, for
// the worst n in 1..Tv: the GEMMs' split partials and the attention's
// partial records depend on the row count.  Memoised per shape.
static size_t sel_scratch_floats(const wam_config& c, int Tv) {
  static std::mutex mu;
  static std::map<std::array<int, 6>, size_t> memo;
  const std::array<int, 6> key{c.d_video, c.n_heads, c.head_dim, c.mlp_ratio, (int)c.dtype, Tv};
  {
    std::lock_guard<std::mutex> g(mu);
    auto it = memo.find(key);
    if (it != memo.end()) return it->second;
  }
  const bool bf = c.dtype == WAM_BF16;
  const int D = c.n_heads * c.head_dim, dv = c.d_video, r = c.mlp_ratio;
  size_t v = 0;
  for (int n = 1; n <= Tv; ++n) {
    v = std::max(v, qkv_ws_floats(bf, n, c.n_heads, c.head_dim, dv));
    v = std::max(v, gemm_ws_floats(bf, n, dv, D));
    v = std::max(v, gemm_ws_floats(bf, n, r * dv, dv));
    v = std::max(v, gemm_ws_floats(bf, n, dv, r * dv));
    v = std::max(v, attention_ws_floats(bf, 1, c.n_heads, c.head_dim, n, Tv, 0));
  }
  std::lock_guard<std::mutex> g(mu);
  memo[key] = v;
  return v;
}

static size_t mod_rows_action(const wam_config& c) { return (size_t)c.n_blocks * 6 * c.d_action + 2 * c.d_action; }

// with_video = false: no video-expert buffers (the targets call reads a
// finished cache); Tv still sizes the action attention's key split.
// selective = true: the video buffers also serve a pass over any number of
// active rows of one sample, plus the active-token index list.
// action_only = true: no video-expert buffers at all (not even its
// conditioning), every action buffer sized exactly as with the video expert:
// the layout of one action step in the fixed scratch of
// wam_action_step_noalloc.
static WsLayout ws_layout(const wam_config& c, int B, int Tv, int Ta, int S, bool with_video = true,
                          bool selective = false, bool action_only = false) {
  WsLayout L;
  const bool bf = c.dtype == WAM_BF16;
  const size_t es = bf ? 2 : 4, f = 4;
  const int D = c.n_heads * c.head_dim, dv = c.d_video, da = c.d_action, r = c.mlp_ratio;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = align256(off);
    off = o + bytes;
    return o;
  };
  const size_t Mv = with_video && !action_only ? (size_t)B * Tv : 0, Ma = (size_t)B * Ta;
  const size_t vc = action_only ? 0 : 1;  // the video conditioning buffers
  L.v_e = take(vc * c.t_freq_dim * f);
  L.v_h1 = take(vc * dv * f);
  L.v_c = take(vc * dv * f);
  L.v_mod = take(vc * c.n_blocks * 6 * dv * f);
  L.v_x = take(Mv * dv * f);
  L.v_h = take(Mv * dv * es);
  L.v_q = take(Mv * D * es);
  L.v_o = take(Mv * D * es);
  L.v_g = take(Mv * r * dv * es);
  size_t vp = 0;
  if (Mv > 0) {
    vp = std::max(vp, qkv_ws_floats(bf, (int)Mv, c.n_heads, c.head_dim, dv));
    vp = std::max(vp, gemm_ws_floats(bf, (int)Mv, dv, D));
    vp = std::max(vp, gemm_ws_floats(bf, (int)Mv, r * dv, dv));
    vp = std::max(vp, gemm_ws_floats(bf, (int)Mv, dv, r * dv));
    vp = std::max(vp, attention_ws_floats(bf, B, c.n_heads, c.head_dim, Tv, Tv, 0));
    if (selective) vp = std::max(vp, sel_scratch_floats(c, Tv));
  }
  L.v_part = take(vp * f);
  L.a_e = take((size_t)S * c.t_freq_dim * f);
  L.a_h1 = take((size_t)S * da * f);
  L.a_c = take((size_t)S * da * f);
  L.a_mod = take((size_t)S * mod_rows_action(c) * f);
  L.a_y = take(Ma * da * f);
  L.a_h = take(Ma * da * es);
  L.a_q = take(Ma * D * es);
  L.a_k = take(Ma * D * es);
  L.a_v = take(Ma * D * es);
  L.a_o = take(Ma * D * es);
  L.a_g = take(Ma * r * da * es);
  size_t ap = 0;
  ap = std::max(ap, qkv_ws_floats(bf, (int)Ma, c.n_heads, c.head_dim, da));
  ap = std::max(ap, gemm_ws_floats(bf, (int)Ma, da, D));
  ap = std::max(ap, gemm_ws_floats(bf, (int)Ma, r * da, da));
  ap = std::max(ap, gemm_ws_floats(bf, (int)Ma, da, r * da));
  L.a_part = take(ap * f);
  // without the video expert (rollouts of one observation) every sample reads one shared cache
  L.a_attn = take(attention_ws_floats(bf, B, c.n_heads, c.head_dim, Ta, Ta, Tv, with_video ? 0 : 1) * f);
  L.a_cur = take(Ma * c.action_dim * f);
  L.g_at = take(with_video ? 0 : Ma * c.action_dim * f);
  L.g_alt = take(with_video ? 0 : Ma * c.action_dim * f);
  L.r_idx = take(selective ? (size_t)Tv * sizeof(int) : 0);
  L.r_count = take(selective ? 16 : 0);
  L.total = align256(off);
  return L;
}

static int check_sizes(const wam_model* m, int B, int Tv, int Ta, int S) {
  const wam_config& c = m->cfg;
  if (B < 1 || B > c.max_batch) return fail(WAM_ERR_SHAPE, "B must be in [1, max_batch]");
  if (Tv < 0 || Tv > c.max_video_tokens) return fail(WAM_ERR_SHAPE, "T_v must be in [0, max_video_tokens]");
  if (Ta < 1 || Ta > c.max_action_tokens) return fail(WAM_ERR_SHAPE, "T_a must be in [1, max_action_tokens]");
  if (S < 1 || S > c.max_steps) return fail(WAM_ERR_SHAPE, "S must be in [1, max_steps]");
  if (c.rope_width > 0 && Tv % (c.rope_height * c.rope_width))
    return fail(WAM_ERR_SHAPE, "T_v must be a whole number of rope_height x rope_width frames");
  return WAM_OK;
}

extern "C" size_t wam_kv_cache_bytes(const wam_model* m, int B, int T_v) {
  if (!m || B < 1 || B > m->cfg.max_batch || T_v < 0 || T_v > m->cfg.max_video_tokens) return 0;
  const size_t es = m->cfg.dtype == WAM_F32 ? 4 : 2;
  return (size_t)m->cfg.n_blocks * 2 * B * m->cfg.n_heads * T_v * m->cfg.head_dim * es;
}

extern "C" size_t wam_workspace_bytes(const wam_model* m, int B, int T_v, int T_a, int S) {
  if (!m) return 0;
  std::string keep = g_err;
  int rc = check_sizes(m, B, T_v, T_a, S);
  g_err = keep;
  if (rc != WAM_OK) return 0;
  return ws_layout(m->cfg, B, T_v, T_a, S).total;
}

// ============================================================================
// enqueue helpers (arguments already validated)
// ============================================================================
template <class T>
struct Run {
  const wam_model* md;
  const wam_config& c;
  uint8_t* ws;
  WsLayout L;
  int B, Tv, Ta;
  int D;
  int Bkv;  // samples in the KV cache (B, or 1 when one observation serves every sample)
  // Per-sample mode (teacher-anchored targets): every action sample has its
  // own time, so its modulation vectors (one conditioning entry per sample)
  // and its Euler times tg / dtg are per sample, and all samples read the
  // one observation's video cache.
  bool per_sample = false;
  TList tg{}, dtg{};

  Run(const wam_model* m, void* ws_, int B_, int Tv_, int Ta_, int S, bool with_video = true, int Bkv_ = -1,
      bool selective = false, bool action_only = false)
      : md(m), c(m->cfg), ws((uint8_t*)ws_),
        L(ws_layout(m->cfg, B_, Tv_, Ta_, S, with_video, selective, action_only)), B(B_), Tv(Tv_), Ta(Ta_),
        D(m->cfg.n_heads * m->cfg.head_dim), Bkv(Bkv_ < 0 ? B_ : Bkv_) {}

  template <class U>
  U* p(size_t off) const { return (U*)(ws + off); }
  static const T* w(const void* x) { return (const T*)x; }

  T* kslab(void* kv, int i) const {
    return (T*)kv + (size_t)i * 2 * Bkv * c.n_heads * Tv * c.head_dim;
  }
  T* vslab(void* kv, int i) const { return kslab(kv, i) + (size_t)Bkv * c.n_heads * Tv * c.head_dim; }

  // c(t) for every t of the list, then every block's six modulation vectors
  // in one pass over the adaLN weights (rows = all blocks' adaLN rows).
  hipError_t conditioning(const ExpertW& e, int d, const TList& ts, size_t o_e, size_t o_h1, size_t o_c, size_t o_mod,
                          size_t mod_rows, hipStream_t s) const {
    hipError_t err = launch_temb(ts, c.t_freq_dim, p<float>(o_e), s);
    const int jmax_t = std::min(16, 16384 / std::max(c.t_freq_dim, d));
    for (int j0 = 0; err == hipSuccess && j0 < ts.n; j0 += jmax_t) {
      const int J = std::min(jmax_t, ts.n - j0);
      err = launch_gemv<T>(w(e.t1_w), d, c.t_freq_dim, p<float>(o_e) + (size_t)j0 * c.t_freq_dim, J, 0, w(e.t1_b), 1,
                           p<float>(o_h1) + (size_t)j0 * d, d, s);
      if (err == hipSuccess)
        err = launch_gemv<T>(w(e.t2_w), d, d, p<float>(o_h1) + (size_t)j0 * d, J, 0, w(e.t2_b), 0,
                             p<float>(o_c) + (size_t)j0 * d, d, s);
      if (err == hipSuccess)
        err = launch_gemv<T>(w(e.ada_w), (int)mod_rows, d, p<float>(o_c) + (size_t)j0 * d, J, 1, w(e.ada_b), 0,
                             p<float>(o_mod) + (size_t)j0 * mod_rows, (int)mod_rows, s);
    }
    return err;
  }

  hipError_t video_prologue(const void* video, float t_v, hipStream_t s) const {
    TList ts{};
    ts.t[0] = t_v;
    ts.n = 1;
    hipError_t e = conditioning(md->vid, c.d_video, ts, L.v_e, L.v_h1, L.v_c, L.v_mod, (size_t)c.n_blocks * 6 * c.d_video, s);
    if (e != hipSuccess) return e;
    return launch_to_f32<T>((const T*)video, (size_t)B * Tv * c.d_video, p<float>(L.v_x), s);
  }

  // one video block; `ev` (if any) is recorded right after the q|k|v projection.
  // Every block runs P, Attn and R, as the schedule lists them (RealtimeWAM
  // digest, Method steps, inference).  kv_only: stop after the projection;
  // set only for the last block, and only when the caller of an inference
  // asks for it (WAM_VIDEO_KV_ONLY_LAST): that block's attention and MLP feed
  // only the video hidden state, which the action expert never reads.
  hipError_t video_block(int i, void* kv, hipEvent_t ev, hipStream_t s, bool kv_only = false) const {
    const int dv = c.d_video, M = B * Tv, H = c.n_heads, dh = c.head_dim, r = c.mlp_ratio;
    const BlockW& bw = md->vid.blk[i];
    const float* mod = p<float>(L.v_mod) + (size_t)i * 6 * dv;
    float* x = p<float>(L.v_x);
    T* h = p<T>(L.v_h);
    T* q = p<T>(L.v_q);
    T* o = p<T>(L.v_o);
    T* g = p<T>(L.v_g);
    float* part = p<float>(L.v_part);
    T* K = kslab(kv, i);
    T* V = vslab(kv, i);
    hipError_t e = launch_delay(md->delay_video_us, s);  // debug hook: nothing unless set
    if (e == hipSuccess) e = launch_ln_mod<T>(x, M, dv, mod, mod + dv, c.ln_eps, h, s);
    if (e == hipSuccess) e = launch_qkv<T>(h, M, dv, w(bw.qkv_w), w(bw.qkv_b), Tv, H, dh, q, K, V, part, s);
    if (e == hipSuccess && (c.qk_norm || c.rope_width))
      e = launch_qk_norm_rope<T>(q, w(bw.qn_g), K, w(bw.kn_g), B, H, Tv, dh, c.ln_eps, c.rope_height, c.rope_width, s);
    if (e == hipSuccess && ev) e = hipEventRecord(ev, s);
    if (e != hipSuccess || kv_only) return e;
    // At its end the attention pulls this block's fc2 weights out of HBM into
    // the Infinity Cache: read cold, fc2 took ~7 us longer in the model.
    AttnPrefetch pf;
    pf.p = w(bw.fc2_w);
    pf.bytes = prefetch_bytes((size_t)r * dv * dv * sizeof(T));
    e = launch_attention<T>(q, K, V, Tv, nullptr, nullptr, 0, B, H, dh, Tv, o, part, s, 0, pf);
    if (e == hipSuccess)
      e = launch_gemm<T>(o, D, w(bw.o_w), D, M, dv, D, EpiGateRes<T>{x, dv, mod + 2 * dv, w(bw.o_b)}, part, s);
    if (e == hipSuccess) e = launch_ln_mod<T>(x, M, dv, mod + 3 * dv, mod + 4 * dv, c.ln_eps, h, s);
    if (e == hipSuccess)
      e = launch_gemm<T>(h, dv, w(bw.fc1_w), dv, M, r * dv, dv, EpiGelu<T>{g, r * dv, w(bw.fc1_b)}, part, s);
    if (e == hipSuccess)
      e = launch_gemm<T>(g, r * dv, w(bw.fc2_w), r * dv, M, dv, r * dv, EpiGateRes<T>{x, dv, mod + 5 * dv, w(bw.fc2_b)},
                         part, s);
    return e;
  }

  // Selective reuse (one sample): the n active tokens idx[0..n) of the new
  // observation start their hidden rows; block i recomputes only them, their
  // K and V land in rows idx of cache slab i (the other rows keep the
  // previous observation's), and their queries attend over all Tv keys.
  hipError_t video_prologue_rows(const void* video, float t_v, const int* idx, int n, hipStream_t s) const {
    TList ts{};
    ts.t[0] = t_v;
    ts.n = 1;
    hipError_t e = conditioning(md->vid, c.d_video, ts, L.v_e, L.v_h1, L.v_c, L.v_mod, (size_t)c.n_blocks * 6 * c.d_video, s);
    if (e != hipSuccess) return e;
    return launch_gather_rows<T>((const T*)video, idx, n, c.d_video, p<float>(L.v_x), s);
  }

  hipError_t video_block_rows(int i, void* kv, const int* idx, int n, hipEvent_t ev, hipStream_t s,
                              bool kv_only = false) const {
    const int dv = c.d_video, H = c.n_heads, dh = c.head_dim, r = c.mlp_ratio;
    const BlockW& bw = md->vid.blk[i];
    const float* mod = p<float>(L.v_mod) + (size_t)i * 6 * dv;
    float* x = p<float>(L.v_x);
    T* h = p<T>(L.v_h);
    T* q = p<T>(L.v_q);
    T* o = p<T>(L.v_o);
    T* g = p<T>(L.v_g);
    float* part = p<float>(L.v_part);
    T* K = kslab(kv, i);
    T* V = vslab(kv, i);
    // K-split gated-residual GEMMs also apply the LayerNorm after them (a
    // function of the shapes only, as in the action blocks); fc2's is the
    // next block's first, so this block's was done by the previous one
    const bool bf = c.dtype == WAM_BF16;
    const bool fuse_wo = gemm_gateres_ln_fusable(bf, n, dv, D);
    const bool fuse_fc2 = gemm_gateres_ln_fusable(bf, n, dv, r * dv);
    hipError_t e = launch_delay(md->delay_video_us, s);  // debug hook: nothing unless set
    if (e == hipSuccess && !(fuse_fc2 && i > 0)) e = launch_ln_mod<T>(x, n, dv, mod, mod + dv, c.ln_eps, h, s);
    if (e == hipSuccess) e = launch_qkv<T>(h, n, dv, w(bw.qkv_w), w(bw.qkv_b), n, H, dh, q, K, V, part, s, idx, Tv);
    if (e == hipSuccess && ev) e = hipEventRecord(ev, s);
    if (e != hipSuccess || kv_only) return e;
    e = launch_attention<T>(q, K, V, Tv, nullptr, nullptr, 0, 1, H, dh, n, o, part, s);
    const EpiGateRes<T> epi_o{x, dv, mod + 2 * dv, w(bw.o_b)};
    if (e == hipSuccess && fuse_wo)
      e = launch_gemm_gateres_ln<T>(o, D, w(bw.o_w), D, n, dv, D, epi_o, mod + 3 * dv, mod + 4 * dv, c.ln_eps, h, part, s);
    if (e == hipSuccess && !fuse_wo) e = launch_gemm<T>(o, D, w(bw.o_w), D, n, dv, D, epi_o, part, s);
    if (e == hipSuccess && !fuse_wo) e = launch_ln_mod<T>(x, n, dv, mod + 3 * dv, mod + 4 * dv, c.ln_eps, h, s);
    if (e == hipSuccess)
      e = launch_gemm<T>(h, dv, w(bw.fc1_w), dv, n, r * dv, dv, EpiGelu<T>{g, r * dv, w(bw.fc1_b)}, part, s);
    const EpiGateRes<T> epi_2{x, dv, mod + 5 * dv, w(bw.fc2_b)};
    const float* mod_next = mod + 6 * dv;  // block i + 1's vectors
    if (e == hipSuccess && fuse_fc2 && i + 1 < c.n_blocks)
      e = launch_gemm_gateres_ln<T>(g, r * dv, w(bw.fc2_w), r * dv, n, dv, r * dv, epi_2, mod_next, mod_next + dv,
                                    c.ln_eps, h, part, s);
    else if (e == hipSuccess)
      e = launch_gemm<T>(g, r * dv, w(bw.fc2_w), r * dv, n, dv, r * dv, epi_2, part, s);
    return e;
  }

  hipError_t action_prologue(const TList& ts, hipStream_t s) const {
    return conditioning(md->act, c.d_action, ts, L.a_e, L.a_h1, L.a_c, L.a_mod, mod_rows_action(c), s);
  }

  hipError_t action_begin(const float* a_in, hipStream_t s) const {
    return launch_action_in<T>(a_in, B * Ta, c.action_dim, w(md->in_w), w(md->in_b), c.d_action, p<float>(L.a_y), s);
  }

  // block i of the action pass for flow-time index j; waits on `ev` (if any)
  // immediately before the attention that consumes video block i's cache
  hipError_t action_block(int j, int i, const void* kv, hipEvent_t ev, hipStream_t s) const {
    const int da = c.d_action, M = B * Ta, H = c.n_heads, dh = c.head_dim, r = c.mlp_ratio;
    const BlockW& bw = md->act.blk[i];
    // per-sample mode: sample b's vectors sit at + b * ms (the step index is not used)
    const size_t ms = per_sample ? mod_rows_action(c) : 0;
    const float* mod = p<float>(L.a_mod) + (per_sample ? 0 : (size_t)j * mod_rows_action(c)) + (size_t)i * 6 * da;
    float* y = p<float>(L.a_y);
    T* h = p<T>(L.a_h);
    T* q = p<T>(L.a_q);
    T* k = p<T>(L.a_k);
    T* v = p<T>(L.a_v);
    T* o = p<T>(L.a_o);
    T* g = p<T>(L.a_g);
    float* part = p<float>(L.a_part);
    // W_o's and fc2's split reductions also apply the LayerNorm that
    // follows them where the shapes allow (a function of the shapes only,
    // so every schedule takes the same path); fc2's is then the next
    // block's first LayerNorm, and this block's was done by the previous one
    const bool bf = c.dtype == WAM_BF16;
    const bool fuse_wo = gemm_gateres_ln_fusable(bf, M, da, D);
    const bool fuse_fc2 = gemm_gateres_ln_fusable(bf, M, da, r * da);
    hipError_t e = hipSuccess;
    if (!(fuse_fc2 && i > 0)) e = launch_ln_mod<T>(y, M, da, mod, mod + da, c.ln_eps, h, s, Ta, ms);
    if (e == hipSuccess) e = launch_qkv<T>(h, M, da, w(bw.qkv_w), w(bw.qkv_b), Ta, H, dh, q, k, v, part, s);
    if (e == hipSuccess && c.qk_norm)  // action tokens: normalised, never rotated
      e = launch_qk_norm_rope<T>(q, w(bw.qn_g), k, w(bw.kn_g), B, H, Ta, dh, c.ln_eps, 0, 0, s);
    if (e == hipSuccess && ev) e = hipStreamWaitEvent(s, ev, 0);
    if (e == hipSuccess) e = launch_delay(md->delay_action_us, s);  // debug hook: nothing unless set
    if (e == hipSuccess)
      e = launch_attention<T>(q, k, v, Ta, kslab((void*)kv, i), vslab((void*)kv, i), Tv, B, H, dh, Ta, o,
                              p<float>(L.a_attn), s, Bkv == 1 && B > 1);
    const EpiGateRes<T> epi_o{y, da, mod + 2 * da, w(bw.o_b), Ta, ms};
    if (e == hipSuccess && fuse_wo)
      e = launch_gemm_gateres_ln<T>(o, D, w(bw.o_w), D, M, da, D, epi_o, mod + 3 * da, mod + 4 * da, c.ln_eps, h, part,
                                    s, Ta, ms);
    if (e == hipSuccess && !fuse_wo) e = launch_gemm<T>(o, D, w(bw.o_w), D, M, da, D, epi_o, part, s);
    if (e == hipSuccess && !fuse_wo) e = launch_ln_mod<T>(y, M, da, mod + 3 * da, mod + 4 * da, c.ln_eps, h, s, Ta, ms);
    if (e == hipSuccess)
      e = launch_gemm<T>(h, da, w(bw.fc1_w), da, M, r * da, da, EpiGelu<T>{g, r * da, w(bw.fc1_b)}, part, s);
    const EpiGateRes<T> epi_2{y, da, mod + 5 * da, w(bw.fc2_b), Ta, ms};
    const float* mod_next = mod + 6 * da;  // block i + 1's vectors (same layout for every step / sample)
    if (e == hipSuccess && fuse_fc2 && i + 1 < c.n_blocks)
      e = launch_gemm_gateres_ln<T>(g, r * da, w(bw.fc2_w), r * da, M, da, r * da, epi_2, mod_next, mod_next + da,
                                    c.ln_eps, h, part, s, Ta, ms);
    else if (e == hipSuccess)
      e = launch_gemm<T>(g, r * da, w(bw.fc2_w), r * da, M, da, r * da, epi_2, part, s);
    return e;
  }

  hipError_t action_end(int j, const float* a_in, float t_cur, float dt, float* a_next, float* v_out, float* f_out,
                        hipStream_t s) const {
    const float* modf = p<float>(L.a_mod) + (per_sample ? 0 : (size_t)j * mod_rows_action(c)) +
                        (size_t)c.n_blocks * 6 * c.d_action;
    if (per_sample)
      return launch_final_euler<T>(p<float>(L.a_y), B * Ta, c.d_action, modf, w(md->out_w), w(md->out_b),
                                   c.action_dim, c.ln_eps, a_in, 0.0f, 0.0f, a_next, v_out, f_out, s, Ta,
                                   mod_rows_action(c), &tg, &dtg);
    return launch_final_euler<T>(p<float>(L.a_y), B * Ta, c.d_action, modf, w(md->out_w), w(md->out_b), c.action_dim,
                                 c.ln_eps, a_in, dt, t_cur, a_next, v_out, f_out, s);
  }

  hipError_t action_pass(int j, const void* kv, const float* a_in, float t_cur, float dt, float* a_next, float* v_out,
                         float* f_out, hipStream_t s) const {
    hipError_t e = action_begin(a_in, s);
    for (int i = 0; e == hipSuccess && i < c.n_blocks; ++i) e = action_block(j, i, kv, nullptr, s);
    if (e == hipSuccess) e = action_end(j, a_in, t_cur, dt, a_next, v_out, f_out, s);
    return e;
  }
};

static int hip_fail(hipError_t e, const char* where) {
  return fail(WAM_ERR_HIP, std::string(where) + ": " + hipGetErrorString(e));
}

// ============================================================================
// entry points
// ============================================================================
template <class T>
static int video_forward_t(wam_model* m, const void* video, int B, int Tv, float t_v, void* kv, float* hidden, void* ws,
                           hipStream_t s) {
  Run<T> r(m, ws, B, Tv, 1, 1);
  hipError_t e = r.video_prologue(video, t_v, s);
  const int N = m->cfg.n_blocks;
  for (int i = 0; e == hipSuccess && i < N; ++i) e = r.video_block(i, kv, nullptr, s);
  if (e == hipSuccess && hidden && Tv > 0)
    e = hipMemcpyAsync(hidden, r.template p<float>(r.L.v_x), (size_t)B * Tv * m->cfg.d_video * sizeof(float),
                       hipMemcpyDeviceToDevice, s);
  return e == hipSuccess ? WAM_OK : hip_fail(e, "wam_video_forward");
}

extern "C" int wam_video_forward(wam_model* m, const void* video_dev, int B, int T_v, float t_v, void* kv_dev,
                                 float* hidden_dev, void* ws_dev, void* stream) {
  if (!m) return fail(WAM_ERR_NULL, "model is NULL");
  int rc = check_sizes(m, B, T_v, 1, 1);
  if (rc != WAM_OK) return rc;
  if ((T_v > 0 && (!video_dev || !kv_dev)) || !ws_dev) return fail(WAM_ERR_NULL, "video, kv and ws must be non-NULL");
  if (!aligned16(video_dev) || !aligned16(kv_dev) || !aligned16(ws_dev) || !aligned16(hidden_dev))
    return fail(WAM_ERR_ALIGN, "device buffers must be 16-byte aligned");
  if (!(t_v >= 0.0f && t_v <= 1.0f)) return fail(WAM_ERR_GRID, "t_v must be in [0, 1]");
  hipStream_t s = (hipStream_t)stream;
  return m->cfg.dtype == WAM_BF16 ? video_forward_t<bf16_t>(m, video_dev, B, T_v, t_v, kv_dev, hidden_dev, ws_dev, s)
                                  : video_forward_t<float>(m, video_dev, B, T_v, t_v, kv_dev, hidden_dev, ws_dev, s);
}

template <class T>
static int action_step_t(wam_model* m, const void* kv, int B, int Tv, int Ta, const float* a, float t_cur, float t_next,
                         float* a_next, float* v, float* f, void* ws, hipStream_t s, bool action_only = false) {
  Run<T> r(m, ws, B, Tv, Ta, 1, true, -1, false, action_only);
  TList ts{};
  ts.t[0] = t_cur;
  ts.n = 1;
  hipError_t e = r.action_prologue(ts, s);
  if (e == hipSuccess) e = r.action_pass(0, kv, a, t_cur, t_cur - t_next, a_next, v, f, s);
  return e == hipSuccess ? WAM_OK : hip_fail(e, "wam_action_step");
}

extern "C" int wam_action_step(wam_model* m, const void* kv_dev, int B, int T_v, int T_a, const float* a_dev,
                               float t_cur, float t_next, float* a_next_dev, float* v_dev, float* endpoint_dev,
                               void* ws_dev, void* stream) {
  if (!m) return fail(WAM_ERR_NULL, "model is NULL");
  int rc = check_sizes(m, B, T_v, T_a, 1);
  if (rc != WAM_OK) return rc;
  if ((T_v > 0 && !kv_dev) || !a_dev || !a_next_dev || !ws_dev)
    return fail(WAM_ERR_NULL, "kv, a, a_next and ws must be non-NULL");
  if (!aligned16(kv_dev) || !aligned16(ws_dev)) return fail(WAM_ERR_ALIGN, "kv and ws must be 16-byte aligned");
  if (!(t_cur > t_next && t_next >= 0.0f && t_cur <= 1.0f))
    return fail(WAM_ERR_GRID, "need 0 <= t_next < t_cur <= 1");
  hipStream_t s = (hipStream_t)stream;
  return m->cfg.dtype == WAM_BF16
             ? action_step_t<bf16_t>(m, kv_dev, B, T_v, T_a, a_dev, t_cur, t_next, a_next_dev, v_dev, endpoint_dev, ws_dev, s)
             : action_step_t<float>(m, kv_dev, B, T_v, T_a, a_dev, t_cur, t_next, a_next_dev, v_dev, endpoint_dev, ws_dev, s);
}

extern "C" int wam_action_step_noalloc(wam_model* m, const void* kv_dev, int B, int T_v, int T_a, const float* a_dev,
                                       float t_cur, float t_next, float* a_next_dev, float* v_dev,
                                       float* endpoint_dev, void* stream) {
  if (!m) return fail(WAM_ERR_NULL, "model is NULL");
  int rc = check_sizes(m, B, T_v, T_a, 1);
  if (rc != WAM_OK) return rc;
  if ((T_v > 0 && !kv_dev) || !a_dev || !a_next_dev) return fail(WAM_ERR_NULL, "kv, a and a_next must be non-NULL");
  if (!aligned16(kv_dev)) return fail(WAM_ERR_ALIGN, "kv must be 16-byte aligned");
  if (!(t_cur > t_next && t_next >= 0.0f && t_cur <= 1.0f))
    return fail(WAM_ERR_GRID, "need 0 <= t_next < t_cur <= 1");
  const size_t need = ws_layout(m->cfg, B, T_v, T_a, 1, true, false, true).total;
  if (need > (size_t)WAM_NOALLOC_SCRATCH_BYTES)
    return fail(WAM_ERR_SHAPE, "wam_action_step_noalloc: these sizes need " + std::to_string(need) +
                                   " bytes of scratch, more than its " + std::to_string(WAM_NOALLOC_SCRATCH_BYTES));
  void* ws = scratch_of(m->device);
  if (!ws) return fail(WAM_ERR_HIP, "wam_action_step_noalloc: no scratch address for the model's device");
  hipStream_t s = (hipStream_t)stream;
  return m->cfg.dtype == WAM_BF16
             ? action_step_t<bf16_t>(m, kv_dev, B, T_v, T_a, a_dev, t_cur, t_next, a_next_dev, v_dev, endpoint_dev, ws,
                                     s, true)
             : action_step_t<float>(m, kv_dev, B, T_v, T_a, a_dev, t_cur, t_next, a_next_dev, v_dev, endpoint_dev, ws,
                                    s, true);
}

// ============================================================================
// selective reuse of the video cache across consecutive observations
// ============================================================================
extern "C" size_t wam_reuse_workspace_bytes(const wam_model* m, int T_v, int T_a, int S) {
  if (!m || T_v < 1 || T_v > m->cfg.max_video_tokens || T_a < 1 || T_a > m->cfg.max_action_tokens || S < 1 ||
      S > m->cfg.max_steps)
    return 0;
  return ws_layout(m->cfg, 1, T_v, T_a, S, true, true).total;
}

static int check_reuse_args(const wam_model* m, const void* vn, const void* vp, int T_v, float tau) {
  if (!m) return fail(WAM_ERR_NULL, "model is NULL");
  if (!vn || !vp) return fail(WAM_ERR_NULL, "video_new and video_prev must be non-NULL");
  if (T_v < 1 || T_v > m->cfg.max_video_tokens) return fail(WAM_ERR_SHAPE, "T_v must be in [1, max_video_tokens]");
  if (!(tau >= 0.0f && tau <= 3.0e38f)) return fail(WAM_ERR_GRID, "tau must be finite and >= 0");
  return WAM_OK;
}

extern "C" int wam_select_tokens(wam_model* m, const void* video_new_dev, const void* video_prev_dev, int T_v,
                                 float tau, int* idx_dev, int* count_dev, void* stream) {
  int rc = check_reuse_args(m, video_new_dev, video_prev_dev, T_v, tau);
  if (rc != WAM_OK) return rc;
  if (!idx_dev || !count_dev) return fail(WAM_ERR_NULL, "idx and count must be non-NULL");
  if (((uintptr_t)idx_dev & 3) || ((uintptr_t)count_dev & 3)) return fail(WAM_ERR_ALIGN, "idx and count must be 4-byte aligned");
  const float tau2 = tau * tau;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = m->cfg.dtype == WAM_BF16
                     ? launch_select_tokens<bf16_t>((const bf16_t*)video_new_dev, (const bf16_t*)video_prev_dev, T_v,
                                                    m->cfg.d_video, tau2, idx_dev, count_dev, s)
                     : launch_select_tokens<float>((const float*)video_new_dev, (const float*)video_prev_dev, T_v,
                                                   m->cfg.d_video, tau2, idx_dev, count_dev, s);
  return e == hipSuccess ? WAM_OK : hip_fail(e, "wam_select_tokens");
}

template <class T>
static int video_forward_reuse_t(wam_model* m, const void* vn, const void* vp, int Tv, float t_v, float tau, void* kv,
                                 float* hidden, int* n_active, void* ws, hipStream_t s) {
  Run<T> r(m, ws, 1, Tv, 1, 1, true, -1, true);  // the layout of wam_reuse_workspace_bytes(T_v, 1, 1)
  int* idx = r.template p<int>(r.L.r_idx);
  int* cnt = r.template p<int>(r.L.r_count);
  hipError_t e = launch_select_tokens<T>((const T*)vn, (const T*)vp, Tv, m->cfg.d_video, tau * tau, idx, cnt, s);
  int na = 0;
  if (e == hipSuccess) e = hipMemcpyAsync(&na, cnt, sizeof(int), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);  // the launches below are sized by the count
  if (e != hipSuccess) return hip_fail(e, "wam_video_forward_reuse");
  if (na < 0 || na > Tv) return fail(WAM_ERR_HIP, "wam_video_forward_reuse: active count out of range");
  if (n_active) *n_active = na;
  if (na == 0) return WAM_OK;
  e = r.video_prologue_rows(vn, t_v, idx, na, s);
  const int N = m->cfg.n_blocks;
  for (int i = 0; e == hipSuccess && i < N; ++i) e = r.video_block_rows(i, kv, idx, na, nullptr, s);
  if (e == hipSuccess && hidden) e = launch_scatter_rows(r.template p<float>(r.L.v_x), idx, na, m->cfg.d_video, hidden, s);
  return e == hipSuccess ? WAM_OK : hip_fail(e, "wam_video_forward_reuse");
}

// The inference on the new observation with the reused cache: selection
// and one host wait for the count on s_video, then the wavefront schedule
// of wam_infer_cewp with the selective video blocks (event i recorded after
// block i's projection of the active rows).
template <class T>
static int infer_reuse_t(wam_model* m, const void* vn, const void* vp, float tau, const float* a_init, const float* grid,
                         int S, int Tv, int Ta, void* kv, float* hidden, float* a_out, float* v_last, float* f_last,
                         int* n_active, int mode, void* ws, hipStream_t sv, hipStream_t sa) {
  Run<T> r(m, ws, 1, Tv, Ta, S, true, -1, true);
  const int N = m->cfg.n_blocks;
  const bool cut_last = (mode & WAM_VIDEO_KV_ONLY_LAST) != 0;
  mode &= ~WAM_VIDEO_KV_ONLY_LAST;
  int* idx = r.template p<int>(r.L.r_idx);
  int* cnt = r.template p<int>(r.L.r_count);
  if (mode == WAM_SEQUENTIAL) sv = sa;
  hipError_t e = hipEventRecord(m->ev_fork, sa);  // the video stream starts after what is queued on s_action
  if (e == hipSuccess) e = hipStreamWaitEvent(sv, m->ev_fork, 0);
  if (e == hipSuccess) e = launch_select_tokens<T>((const T*)vn, (const T*)vp, Tv, m->cfg.d_video, tau * tau, idx, cnt, sv);
  int na = 0;
  if (e == hipSuccess) e = hipMemcpyAsync(&na, cnt, sizeof(int), hipMemcpyDeviceToHost, sv);
  if (e == hipSuccess) e = hipStreamSynchronize(sv);
  if (e != hipSuccess) return hip_fail(e, "wam_infer_reuse");
  if (na < 0 || na > Tv) return fail(WAM_ERR_HIP, "wam_infer_reuse: active count out of range");
  if (n_active) *n_active = na;
  TList ts{};
  ts.n = S;
  for (int j = 0; j < S; ++j) ts.t[j] = grid[S - j];
  float* a_cur = r.template p<float>(r.L.a_cur);
  auto io = [&](int j, const float** in, float** out, float** vo, float** fo) {
    *in = j == 0 ? a_init : a_cur;
    const bool last = j == S - 1;
    *out = last ? a_out : a_cur;
    *vo = last ? v_last : nullptr;
    *fo = last ? f_last : nullptr;
  };
  if (na > 0) e = r.video_prologue_rows(vn, 0.0f, idx, na, sv);
  if (e == hipSuccess) e = r.action_prologue(ts, sa);
  if (e == hipSuccess) e = r.action_begin(a_init, sa);
  // video block i (recording e_i) is enqueued before the action block waiting on e_i
  for (int i = 0; e == hipSuccess && i < N; ++i) {
    const bool wave = mode == WAM_CEWP && na > 0;
    if (na > 0)
      e = r.video_block_rows(i, kv, idx, na, wave ? m->ev_block[i] : nullptr, sv, cut_last && !hidden && i == N - 1);
    if (e == hipSuccess) e = r.action_block(0, i, kv, wave ? m->ev_block[i] : nullptr, sa);
  }
  {
    const float *in;
    float *out, *vo, *fo;
    io(0, &in, &out, &vo, &fo);
    if (e == hipSuccess) e = r.action_end(0, in, grid[S], grid[S] - grid[S - 1], out, vo, fo, sa);
  }
  if (e == hipSuccess && hidden && na > 0)
    e = launch_scatter_rows(r.template p<float>(r.L.v_x), idx, na, m->cfg.d_video, hidden, sv);
  // the steps after the first read every block's finished cache
  if (e == hipSuccess && sv != sa) e = hipEventRecord(m->ev_join, sv);
  if (e == hipSuccess && sv != sa) e = hipStreamWaitEvent(sa, m->ev_join, 0);
  for (int j = 1; e == hipSuccess && j < S; ++j) {
    const float *in;
    float *out, *vo, *fo;
    io(j, &in, &out, &vo, &fo);
    e = r.action_pass(j, kv, in, grid[S - j], grid[S - j] - grid[S - j - 1], out, vo, fo, sa);
  }
  return e == hipSuccess ? WAM_OK : hip_fail(e, "wam_infer_reuse");
}

extern "C" int wam_video_forward_reuse(wam_model* m, const void* video_new_dev, const void* video_prev_dev, int T_v,
                                       float t_v, float tau, void* kv_dev, float* hidden_dev, int* n_active,
                                       void* ws_dev, void* stream) {
  int rc = check_reuse_args(m, video_new_dev, video_prev_dev, T_v, tau);
  if (rc != WAM_OK) return rc;
  if (m->cfg.qk_norm || m->cfg.rope_width)
    return fail(WAM_ERR_SHAPE, "selective reuse is defined for the base block (no qk_norm / rope)");
  if (!kv_dev || !ws_dev) return fail(WAM_ERR_NULL, "kv and ws must be non-NULL");
  if (!aligned16(video_new_dev) || !aligned16(video_prev_dev) || !aligned16(kv_dev) || !aligned16(ws_dev) ||
      !aligned16(hidden_dev))
    return fail(WAM_ERR_ALIGN, "device buffers must be 16-byte aligned");
  if (!(t_v >= 0.0f && t_v <= 1.0f)) return fail(WAM_ERR_GRID, "t_v must be in [0, 1]");
  hipStream_t s = (hipStream_t)stream;
  return m->cfg.dtype == WAM_BF16
             ? video_forward_reuse_t<bf16_t>(m, video_new_dev, video_prev_dev, T_v, t_v, tau, kv_dev, hidden_dev,
                                             n_active, ws_dev, s)
             : video_forward_reuse_t<float>(m, video_new_dev, video_prev_dev, T_v, t_v, tau, kv_dev, hidden_dev,
                                            n_active, ws_dev, s);
}

// ============================================================================
// teacher-anchored targets (forward only)
// ============================================================================
static bool same_shape(const wam_config& a, const wam_config& b) {
  return a.n_blocks == b.n_blocks && a.d_video == b.d_video && a.d_action == b.d_action && a.n_heads == b.n_heads &&
         a.head_dim == b.head_dim && a.mlp_ratio == b.mlp_ratio && a.t_freq_dim == b.t_freq_dim &&
         a.action_dim == b.action_dim && a.dtype == b.dtype && a.ln_eps == b.ln_eps && a.qk_norm == b.qk_norm &&
         a.rope_height == b.rope_height && a.rope_width == b.rope_width;
}

template <class T>
static int targets_t(const wam_model* teacher, const wam_model* student, const void* kv, int Tv, int R, int Ta,
                     const float* a0, const float* eps, const float* t_host, int K, float* a_t_out, float* u_out,
                     float* f_out, void* ws, hipStream_t s) {
  Run<T> rt(teacher, ws, R, Tv, Ta, R, false, 1);
  Run<T> rs(student, ws, R, Tv, Ta, R, false, 1);
  rt.per_sample = rs.per_sample = true;
  const int N = teacher->cfg.n_blocks, A = teacher->cfg.action_dim, n = R * Ta * A;
  float* a_t = rt.template p<float>(rt.L.g_at);
  float* buf[2] = {rt.template p<float>(rt.L.a_cur), rt.template p<float>(rt.L.g_alt)};
  TList tg{};
  tg.n = R;
  for (int r = 0; r < R; ++r) tg.t[r] = t_host[r];
  hipError_t e = launch_targets_init(a0, eps, n, Ta * A, tg, a_t, a_t_out, s);
  // the teacher's K Euler steps from t_r to 0 on the grid t_r j / K (float32)
  const float* a_in = a_t;
  for (int j = K; e == hipSuccess && j >= 1; --j) {
    TList tj{}, dtj{};
    tj.n = dtj.n = R;
    for (int r = 0; r < R; ++r) {
      const float hi = t_host[r] * (float)j / (float)K, lo = t_host[r] * (float)(j - 1) / (float)K;
      tj.t[r] = hi;
      dtj.t[r] = hi - lo;
    }
    rt.tg = tj;
    rt.dtg = dtj;
    float* a_out = buf[j & 1];
    e = rt.action_prologue(tj, s);
    if (e == hipSuccess) e = rt.action_begin(a_in, s);
    for (int i = 0; e == hipSuccess && i < N; ++i) e = rt.action_block(0, i, kv, nullptr, s);
    if (e == hipSuccess) e = rt.action_end(0, a_in, 0.0f, 0.0f, a_out, nullptr, nullptr, s);
    a_in = a_out;
  }
  if (e == hipSuccess) e = launch_targets_u(a_t, a_in, n, Ta * A, tg, u_out, s);
  // the student's endpoint at (a_t, t_r)
  rs.tg = rs.dtg = tg;
  float* scratch = a_in == buf[0] ? buf[1] : buf[0];
  if (e == hipSuccess) e = rs.action_prologue(tg, s);
  if (e == hipSuccess) e = rs.action_begin(a_t, s);
  for (int i = 0; e == hipSuccess && i < N; ++i) e = rs.action_block(0, i, kv, nullptr, s);
  if (e == hipSuccess) e = rs.action_end(0, a_t, 0.0f, 0.0f, scratch, nullptr, f_out, s);
  return e == hipSuccess ? WAM_OK : hip_fail(e, "wam_teacher_targets");
}

static int check_targets(const wam_model* m, int R, int Tv, int Ta) {
  if (R < 1 || R > WAM_MAX_T || R > m->cfg.max_batch) return fail(WAM_ERR_SHAPE, "R must be in [1, min(64, max_batch)]");
  return check_sizes(m, 1, Tv, Ta, 1);
}

extern "C" size_t wam_targets_workspace_bytes(const wam_model* m, int R, int T_v, int T_a) {
  if (!m) return 0;
  std::string keep = g_err;
  int rc = check_targets(m, R, T_v, T_a);
  g_err = keep;
  if (rc != WAM_OK) return 0;
  return ws_layout(m->cfg, R, T_v, T_a, R, false).total;
}

extern "C" int wam_teacher_targets(wam_model* teacher, wam_model* student, const void* kv_dev, int T_v, int R, int T_a,
                                   const float* a0_dev, const float* eps_dev, const float* t_host, int K,
                                   float* a_t_dev, float* u_dev, float* f_dev, void* ws_dev, void* stream) {
  if (!teacher) return fail(WAM_ERR_NULL, "teacher model is NULL");
  if (!student) student = teacher;
  if (!same_shape(teacher->cfg, student->cfg)) return fail(WAM_ERR_SHAPE, "teacher and student shapes differ");
  int rc = check_targets(teacher, R, T_v, T_a);
  if (rc == WAM_OK) rc = check_targets(student, R, T_v, T_a);
  if (rc != WAM_OK) return rc;
  if ((T_v > 0 && !kv_dev) || !a0_dev || !eps_dev || !t_host || !u_dev || !f_dev || !ws_dev)
    return fail(WAM_ERR_NULL, "kv, a0, eps, t, u, f and ws must be non-NULL");
  if (!aligned16(kv_dev) || !aligned16(ws_dev)) return fail(WAM_ERR_ALIGN, "kv and ws must be 16-byte aligned");
  if (K < 1 || K > 1024) return fail(WAM_ERR_GRID, "K must be in [1, 1024]");
  for (int r = 0; r < R; ++r)
    if (!(t_host[r] > 0.0f && t_host[r] <= 1.0f)) return fail(WAM_ERR_GRID, "every t must lie in (0, 1]");
  hipStream_t s = (hipStream_t)stream;
  return teacher->cfg.dtype == WAM_BF16
             ? targets_t<bf16_t>(teacher, student, kv_dev, T_v, R, T_a, a0_dev, eps_dev, t_host, K, a_t_dev, u_dev,
                                 f_dev, ws_dev, s)
             : targets_t<float>(teacher, student, kv_dev, T_v, R, T_a, a0_dev, eps_dev, t_host, K, a_t_dev, u_dev,
                                f_dev, ws_dev, s);
}

// part: 0 = the whole inference; in wavefront mode 1 = the video expert, the
// first action step and the join, 2 = the later action steps (on s_action).
template <class T>
static int infer_t(wam_model* m, const void* video, const float* a_init, const float* grid, int S, int B, int Tv, int Ta,
                   void* kv, float* a_out, float* v_last, float* f_last, int mode, void* ws, hipStream_t sv,
                   hipStream_t sa, int part = 0) {
  Run<T> r(m, ws, B, Tv, Ta, S);
  const int N = m->cfg.n_blocks;
  const bool cut_last = (mode & WAM_VIDEO_KV_ONLY_LAST) != 0;  // off unless asked for
  mode &= ~WAM_VIDEO_KV_ONLY_LAST;
  TList ts{};
  ts.n = S;
  for (int j = 0; j < S; ++j) ts.t[j] = grid[S - j];  // step j runs at t_{S-j}
  float* a_cur = r.template p<float>(r.L.a_cur);
  auto step_io = [&](int j, const float** in, float** out, float** vo, float** fo) {
    *in = j == 0 ? a_init : a_cur;
    const bool last = j == S - 1;
    *out = last ? a_out : a_cur;
    *vo = last ? v_last : nullptr;
    *fo = last ? f_last : nullptr;
  };
  hipError_t e = hipSuccess;
  if (mode == WAM_SEQUENTIAL) {
    e = r.video_prologue(video, 0.0f, sa);
    for (int i = 0; e == hipSuccess && i < N; ++i) e = r.video_block(i, kv, nullptr, sa, cut_last && i == N - 1);
    if (e == hipSuccess) e = r.action_prologue(ts, sa);
    for (int j = 0; e == hipSuccess && j < S; ++j) {
      const float *in;
      float *out, *vo, *fo;
      step_io(j, &in, &out, &vo, &fo);
      e = r.action_pass(j, kv, in, grid[S - j], grid[S - j] - grid[S - j - 1], out, vo, fo, sa);
    }
  } else if (part == 2) {
    for (int j = 1; e == hipSuccess && j < S; ++j) {
      const float *in;
      float *out, *vo, *fo;
      step_io(j, &in, &out, &vo, &fo);
      e = r.action_pass(j, kv, in, grid[S - j], grid[S - j] - grid[S - j - 1], out, vo, fo, sa);
    }
  } else {
    // fork: the video stream starts after everything already queued on s_action
    e = hipEventRecord(m->ev_fork, sa);
    if (e == hipSuccess) e = hipStreamWaitEvent(sv, m->ev_fork, 0);
    if (e == hipSuccess) e = r.video_prologue(video, 0.0f, sv);
    if (e == hipSuccess) e = r.action_prologue(ts, sa);
    if (e == hipSuccess) e = r.action_begin(a_init, sa);
    // Enqueue order matters for correctness: video block i (which records
    // e_i) is enqueued before the action block that waits on e_i.
    for (int i = 0; e == hipSuccess && i < N; ++i) {
      e = r.video_block(i, kv, m->ev_block[i], sv, cut_last && i == N - 1);
      if (e == hipSuccess) e = r.action_block(0, i, kv, m->ev_block[i], sa);
    }
    {
      const float *in;
      float *out, *vo, *fo;
      step_io(0, &in, &out, &vo, &fo);
      if (e == hipSuccess) e = r.action_end(0, in, grid[S], grid[S] - grid[S - 1], out, vo, fo, sa);
    }
    for (int j = 1; e == hipSuccess && part == 0 && j < S; ++j) {
      const float *in;
      float *out, *vo, *fo;
      step_io(j, &in, &out, &vo, &fo);
      e = r.action_pass(j, kv, in, grid[S - j], grid[S - j] - grid[S - j - 1], out, vo, fo, sa);
    }
    // join: s_action continues only after the whole video expert
    if (e == hipSuccess) e = hipEventRecord(m->ev_join, sv);
    if (e == hipSuccess) e = hipStreamWaitEvent(sa, m->ev_join, 0);
  }
  return e == hipSuccess ? WAM_OK : hip_fail(e, "wam_infer_cewp");
}

static int check_infer_args(wam_model* m, const void* video_dev, const float* a_init_dev, const float* t_grid_host,
                            int S, int B, int T_v, int T_a, void* kv_dev, float* a_out_dev, int mode, void* ws_dev) {
  if (!m) return fail(WAM_ERR_NULL, "model is NULL");
  if (!t_grid_host) return fail(WAM_ERR_NULL, "t_grid_host is NULL");
  if (S < 1) return fail(WAM_ERR_GRID, "S must be >= 1");
  int rc = check_sizes(m, B, T_v, T_a, S);
  if (rc != WAM_OK) return rc;
  if ((T_v > 0 && (!video_dev || !kv_dev)) || !a_init_dev || !a_out_dev || !ws_dev)
    return fail(WAM_ERR_NULL, "video, kv, a_init, a_out and ws must be non-NULL");
  if (!aligned16(video_dev) || !aligned16(kv_dev) || !aligned16(ws_dev))
    return fail(WAM_ERR_ALIGN, "video, kv and ws must be 16-byte aligned");
  const int sched = mode & ~WAM_VIDEO_KV_ONLY_LAST;
  if (sched != WAM_SEQUENTIAL && sched != WAM_CEWP)
    return fail(WAM_ERR_SHAPE, "mode must be WAM_SEQUENTIAL or WAM_CEWP, optionally with WAM_VIDEO_KV_ONLY_LAST");
  for (int j = 0; j <= S; ++j)
    if (!(t_grid_host[j] >= 0.0f && t_grid_host[j] <= 1.0f)) return fail(WAM_ERR_GRID, "t_grid values must be in [0, 1]");
  for (int j = 1; j <= S; ++j)
    if (!(t_grid_host[j] > t_grid_host[j - 1])) return fail(WAM_ERR_GRID, "t_grid must be strictly increasing");
  return WAM_OK;
}

static int infer_dispatch(wam_model* m, const void* video_dev, const float* a_init_dev, const float* t_grid_host, int S,
                          int B, int T_v, int T_a, void* kv_dev, float* a_out_dev, float* v_last_dev, float* f_last_dev,
                          int mode, void* ws_dev, hipStream_t sv, hipStream_t sa, int part = 0) {
  return m->cfg.dtype == WAM_BF16
             ? infer_t<bf16_t>(m, video_dev, a_init_dev, t_grid_host, S, B, T_v, T_a, kv_dev, a_out_dev, v_last_dev,
                               f_last_dev, mode, ws_dev, sv, sa, part)
             : infer_t<float>(m, video_dev, a_init_dev, t_grid_host, S, B, T_v, T_a, kv_dev, a_out_dev, v_last_dev,
                              f_last_dev, mode, ws_dev, sv, sa, part);
}

extern "C" int wam_infer_cewp(wam_model* m, const void* video_dev, const float* a_init_dev, const float* t_grid_host,
                              int S, int B, int T_v, int T_a, void* kv_dev, float* a_out_dev, float* v_last_dev,
                              float* f_last_dev, int mode, void* ws_dev, void* s_video, void* s_action) {
  int rc = check_infer_args(m, video_dev, a_init_dev, t_grid_host, S, B, T_v, T_a, kv_dev, a_out_dev, mode, ws_dev);
  if (rc != WAM_OK) return rc;
  return infer_dispatch(m, video_dev, a_init_dev, t_grid_host, S, B, T_v, T_a, kv_dev, a_out_dev, v_last_dev,
                        f_last_dev, mode, ws_dev, (hipStream_t)s_video, (hipStream_t)s_action);
}

extern "C" int wam_infer_reuse(wam_model* m, const void* video_new_dev, const void* video_prev_dev, float tau,
                               const float* a_init_dev, const float* t_grid_host, int S, int T_v, int T_a, void* kv_dev,
                               float* hidden_dev, float* a_out_dev, float* v_last_dev, float* f_last_dev,
                               int* n_active, int mode, void* ws_dev, void* s_video, void* s_action) {
  int rc = check_reuse_args(m, video_new_dev, video_prev_dev, T_v, tau);
  if (rc != WAM_OK) return rc;
  rc = check_infer_args(m, video_new_dev, a_init_dev, t_grid_host, S, 1, T_v, T_a, kv_dev, a_out_dev, mode, ws_dev);
  if (rc != WAM_OK) return rc;
  if (m->cfg.qk_norm || m->cfg.rope_width)
    return fail(WAM_ERR_SHAPE, "selective reuse is defined for the base block (no qk_norm / rope)");
  if (!aligned16(video_prev_dev) || !aligned16(hidden_dev)) return fail(WAM_ERR_ALIGN, "device buffers must be 16-byte aligned");
  hipStream_t sv = (hipStream_t)s_video, sa = (hipStream_t)s_action;
  return m->cfg.dtype == WAM_BF16
             ? infer_reuse_t<bf16_t>(m, video_new_dev, video_prev_dev, tau, a_init_dev, t_grid_host, S, T_v, T_a, kv_dev,
                                     hidden_dev, a_out_dev, v_last_dev, f_last_dev, n_active, mode, ws_dev, sv, sa)
             : infer_reuse_t<float>(m, video_new_dev, video_prev_dev, tau, a_init_dev, t_grid_host, S, T_v, T_a, kv_dev,
                                    hidden_dev, a_out_dev, v_last_dev, f_last_dev, n_active, mode, ws_dev, sv, sa);
}

// ============================================================================
// captured inference
// ============================================================================
// One captured inference.  In wavefront mode with S > 1 it is two graphs
// launched back to back: the video expert with the first action step and
// the join, then the later action steps captured from s_action alone.  As one
// two-branch graph, those later steps (a single chain of kernels) ran ~12%
// slower than the same kernels launched on one stream (fastwam_s10 on
// MI355X: 25.1 ms against 23.0 ms eager in a closed loop); as a graph of
// their own they run as a plain chain.
struct wam_graph {
  hipGraph_t graph[2] = {nullptr, nullptr};
  hipGraphExec_t exec[2] = {nullptr, nullptr};
};

static int capture(wam_model* m, const void* video_dev, const float* a_init_dev, const float* t_grid_host, int S, int B,
                   int T_v, int T_a, void* kv_dev, float* a_out_dev, float* v_last_dev, float* f_last_dev, int mode,
                   void* ws_dev, hipStream_t sv, hipStream_t sa, int part, hipGraph_t* g_out, hipGraphExec_t* x_out) {
  hipError_t e = hipStreamBeginCapture(sa, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) return hip_fail(e, "hipStreamBeginCapture");
  int rc = infer_dispatch(m, video_dev, a_init_dev, t_grid_host, S, B, T_v, T_a, kv_dev, a_out_dev, v_last_dev,
                          f_last_dev, mode, ws_dev, sv, sa, part);
  std::string enqueue_err = rc != WAM_OK ? g_err : std::string();
  hipGraph_t g = nullptr;
  e = hipStreamEndCapture(sa, &g);  // always end the capture, so the stream stays usable
  if (rc != WAM_OK) {
    if (g) (void)hipGraphDestroy(g);
    return fail(rc, "capture: " + enqueue_err);
  }
  if (e != hipSuccess) return hip_fail(e, "hipStreamEndCapture");
  hipGraphExec_t x = nullptr;
  e = hipGraphInstantiate(&x, g, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    (void)hipGraphDestroy(g);
    return hip_fail(e, "hipGraphInstantiate");
  }
  *g_out = g;
  *x_out = x;
  return WAM_OK;
}

extern "C" int wam_graph_create(wam_model* m, const void* video_dev, const float* a_init_dev, const float* t_grid_host,
                                int S, int B, int T_v, int T_a, void* kv_dev, float* a_out_dev, float* v_last_dev,
                                float* f_last_dev, int mode, void* ws_dev, void* s_video, void* s_action,
                                wam_graph** out) {
  if (!out) return fail(WAM_ERR_NULL, "out is NULL");
  int rc = check_infer_args(m, video_dev, a_init_dev, t_grid_host, S, B, T_v, T_a, kv_dev, a_out_dev, mode, ws_dev);
  if (rc != WAM_OK) return rc;
  const bool wave = (mode & ~WAM_VIDEO_KV_ONLY_LAST) == WAM_CEWP;
  if (!s_action || (wave && !s_video))
    return fail(WAM_ERR_NULL, "graph capture needs non-NULL streams (the null stream cannot be captured)");
  hipStream_t sa = (hipStream_t)s_action, sv = (hipStream_t)s_video;
  wam_graph* wg = new wam_graph();
  const bool split = wave && S > 1;
  for (int k = 0; rc == WAM_OK && k < (split ? 2 : 1); ++k)
    rc = capture(m, video_dev, a_init_dev, t_grid_host, S, B, T_v, T_a, kv_dev, a_out_dev, v_last_dev, f_last_dev,
                 mode, ws_dev, sv, sa, split ? k + 1 : 0, &wg->graph[k], &wg->exec[k]);
  if (rc != WAM_OK) {
    std::string msg = g_err;
    (void)wam_graph_destroy(wg);
    return fail(rc, msg);
  }
  *out = wg;
  return WAM_OK;
}

extern "C" int wam_graph_launch(wam_graph* g, void* stream) {
  if (!g) return fail(WAM_ERR_NULL, "graph is NULL");
  for (int k = 0; k < 2 && g->exec[k]; ++k) {
    hipError_t e = hipGraphLaunch(g->exec[k], (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "hipGraphLaunch");
  }
  return WAM_OK;
}

extern "C" int wam_graph_destroy(wam_graph* g) {
  if (!g) return fail(WAM_ERR_NULL, "graph is NULL");
  for (int k = 0; k < 2; ++k) {
    if (g->exec[k]) (void)hipGraphExecDestroy(g->exec[k]);
    if (g->graph[k]) (void)hipGraphDestroy(g->graph[k]);
  }
  delete g;
  return WAM_OK;
}

// ============================================================================
// single-kernel entry points (wam_ops.h)
// ============================================================================
extern "C" size_t wam_op_gemm_ws_bytes(int dtype, int M, int N, int K) {
  if (M < 1 || N < 1 || K < 1 || (dtype != WAM_F32 && dtype != WAM_BF16)) return 0;
  const bool bf = dtype == WAM_BF16;
  size_t f = gemm_ws_floats(bf, M, N, K);
  // the q|k|v epilogue may run as two GEMMs (q|k, then the transposed values)
  if (N % 3 == 0) f = std::max(f, std::max(gemm_ws_floats(bf, M, 2 * N / 3, K), gemm_ws_floats(bf, N / 3, M, K)));
  return f * sizeof(float);
}

template <class T>
static hipError_t op_gemm_t(int epi, int M, int N, int K, const void* A, const void* W, const void* bias,
                            const float* gate, int dh, void* out, void* ws, hipStream_t s) {
  const T* a = (const T*)A;
  const T* w = (const T*)W;
  const T* b = (const T*)bias;
  float* part = (float*)ws;
  switch (epi) {
    case WAM_EPI_F32:
      return launch_gemm<T>(a, K, w, K, M, N, K, EpiF32<T>{(float*)out, N, b, 0}, part, s);
    case WAM_EPI_GELU:
      return launch_gemm<T>(a, K, w, K, M, N, K, EpiGelu<T>{(T*)out, N, b}, part, s);
    case WAM_EPI_GATE_RES:
      return launch_gemm<T>(a, K, w, K, M, N, K, EpiGateRes<T>{(float*)out, N, gate, b}, part, s);
    default: {
      const int H = N / (3 * dh);
      T* q = (T*)out;
      return launch_qkv<T>(a, M, K, w, b, M, H, dh, q, q + (size_t)M * H * dh, q + (size_t)2 * M * H * dh, part, s);
    }
  }
}

extern "C" int wam_op_gemm(int dtype, int epi, int M, int N, int K, const void* A, const void* W, const void* bias,
                           const float* gate, int head_dim, void* out, void* ws, void* stream) {
  if (dtype != WAM_F32 && dtype != WAM_BF16) return fail(WAM_ERR_DTYPE, "dtype");
  if (epi < WAM_EPI_F32 || epi > WAM_EPI_QKV) return fail(WAM_ERR_SHAPE, "epi must be a wam_epi value");
  if (M < 1 || N < 1 || K < 1) return fail(WAM_ERR_SHAPE, "M, N, K must be >= 1");
  if (dtype == WAM_BF16 && K % 64) return fail(WAM_ERR_SHAPE, "bf16 GEMM needs K % 64 == 0");
  if (epi == WAM_EPI_QKV && (head_dim < 1 || N % (3 * head_dim)))
    return fail(WAM_ERR_SHAPE, "q|k|v epilogue needs N a multiple of 3*head_dim");
  if (!A || !W || !bias || !out || (epi == WAM_EPI_GATE_RES && !gate))
    return fail(WAM_ERR_NULL, "A, W, bias, out (and gate for the residual epilogue) must be non-NULL");
  if (wam_op_gemm_ws_bytes(dtype, M, N, K) > 0 && !ws) return fail(WAM_ERR_NULL, "this shape needs a workspace");
  if (!aligned16(A) || !aligned16(W) || !aligned16(ws) || !aligned16(bias) || !aligned16(gate) || !aligned16(out))
    return fail(WAM_ERR_ALIGN, "A, W, bias, gate, out and ws must be 16-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = dtype == WAM_BF16 ? op_gemm_t<bf16_t>(epi, M, N, K, A, W, bias, gate, head_dim, out, ws, s)
                                   : op_gemm_t<float>(epi, M, N, K, A, W, bias, gate, head_dim, out, ws, s);
  return e == hipSuccess ? WAM_OK : hip_fail(e, "wam_op_gemm");
}

extern "C" size_t wam_op_attention_ws_bytes(int dtype, int B, int H, int dh, int Tq, int L0, int L1) {
  if (B < 1 || H < 1 || Tq < 1 || L0 < 0 || L1 < 0 || L0 + L1 < 1) return 0;
  return attention_ws_floats(dtype == WAM_BF16, B, H, dh, Tq, L0, L1) * sizeof(float);
}

extern "C" int wam_op_attention(int dtype, int B, int H, int dh, int Tq, const void* q, int L0, const void* k0,
                                const void* v0, int L1, const void* k1, const void* v1, void* o, void* ws,
                                void* stream) {
  if (dtype != WAM_F32 && dtype != WAM_BF16) return fail(WAM_ERR_DTYPE, "dtype");
  if (B < 1 || H < 1 || Tq < 1 || L0 < 0 || L1 < 0 || L0 + L1 < 1) return fail(WAM_ERR_SHAPE, "sizes");
  if (dtype == WAM_BF16 ? (dh != 64 && dh != 128) : (dh != 32 && dh != 64 && dh != 128))
    return fail(WAM_ERR_SHAPE, "head_dim");
  if (!q || !o || (L0 > 0 && (!k0 || !v0)) || (L1 > 0 && (!k1 || !v1))) return fail(WAM_ERR_NULL, "buffers");
  if (wam_op_attention_ws_bytes(dtype, B, H, dh, Tq, L0, L1) > 0 && !ws) return fail(WAM_ERR_NULL, "needs workspace");
  if (!aligned16(q) || !aligned16(k0) || !aligned16(v0) || !aligned16(k1) || !aligned16(v1) || !aligned16(o))
    return fail(WAM_ERR_ALIGN, "buffers must be 16-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (dtype == WAM_BF16)
    e = launch_attention<bf16_t>((const bf16_t*)q, (const bf16_t*)k0, (const bf16_t*)v0, L0, (const bf16_t*)k1,
                                 (const bf16_t*)v1, L1, B, H, dh, Tq, (bf16_t*)o, (float*)ws, s);
  else
    e = launch_attention<float>((const float*)q, (const float*)k0, (const float*)v0, L0, (const float*)k1,
                                (const float*)v1, L1, B, H, dh, Tq, (float*)o, (float*)ws, s);
  return e == hipSuccess ? WAM_OK : hip_fail(e, "wam_op_attention");
}

extern "C" int wam_op_ln_modulate(int dtype, int rows, int d, const float* x, const float* shift, const float* scale,
                                  float eps, void* h, void* stream) {
  if (dtype != WAM_F32 && dtype != WAM_BF16) return fail(WAM_ERR_DTYPE, "dtype");
  if (rows < 1 || d < 4 || d % 4 || d > 8192) return fail(WAM_ERR_SHAPE, "rows >= 1, d a multiple of 4 in [4, 8192]");
  if (!x || !shift || !scale || !h) return fail(WAM_ERR_NULL, "buffers");
  if (!aligned16(x) || !aligned16(shift) || !aligned16(scale) || !aligned16(h))
    return fail(WAM_ERR_ALIGN, "buffers must be 16-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = dtype == WAM_BF16 ? launch_ln_mod<bf16_t>(x, rows, d, shift, scale, eps, (bf16_t*)h, s)
                                   : launch_ln_mod<float>(x, rows, d, shift, scale, eps, (float*)h, s);
  return e == hipSuccess ? WAM_OK : hip_fail(e, "wam_op_ln_modulate");
}

extern "C" int wam_op_qk_norm_rope(int dtype, int B, int H, int T, int dh, void* x, const void* gain, float eps,
                                   int rope_height, int rope_width, void* stream) {
  if (dtype != WAM_F32 && dtype != WAM_BF16) return fail(WAM_ERR_DTYPE, "dtype");
  if (B < 1 || H < 1 || T < 1 || (dh != 32 && dh != 64 && dh != 128) || (long long)H * dh > 16384)
    return fail(WAM_ERR_SHAPE, "B, H, T >= 1; dh in {32, 64, 128}; H*dh <= 16384");
  if ((rope_height == 0) != (rope_width == 0) || rope_height < 0 || rope_width < 0 ||
      (rope_width > 0 && T % (rope_height * rope_width)))
    return fail(WAM_ERR_SHAPE, "rope_height and rope_width both 0, or T a multiple of their product");
  if (!x) return fail(WAM_ERR_NULL, "x is NULL");
  if (!(eps > 0.0f)) return fail(WAM_ERR_SHAPE, "eps must be > 0");
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = dtype == WAM_BF16
                     ? launch_qk_norm_rope<bf16_t>((bf16_t*)x, (const bf16_t*)gain, nullptr, nullptr, B, H, T, dh, eps,
                                                   rope_height, rope_width, s)
                     : launch_qk_norm_rope<float>((float*)x, (const float*)gain, nullptr, nullptr, B, H, T, dh, eps,
                                                  rope_height, rope_width, s);
  return e == hipSuccess ? WAM_OK : hip_fail(e, "wam_op_qk_norm_rope");
}
