// C ABI of libk2: argument validation, workspace carving and kernel sequencing.
// Declarations and the contract of every entry point are in include/k2.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <atomic>
#include <climits>
#include <mutex>
#include <initializer_list>
#include <string>
#include <vector>

#include "k2.h"
#include "k2_kernels.h"

using namespace k2;

namespace {

// ---------------------------------------------------------------------------------------------
// Errors
// ---------------------------------------------------------------------------------------------
thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

// ---------------------------------------------------------------------------------------------
// Optional per-kernel event timing
// ---------------------------------------------------------------------------------------------
struct ProfEvent {
  std::string name;
  hipEvent_t a, b;
};
// The one piece of process-wide state: the timing facility below (a diagnostic, off by default).
// The flag is atomic; the event lists and the filter are guarded by g_pm.
std::mutex g_pm;
std::atomic<bool> g_prof{false};
std::string g_pfilter;  // record only kernels of this name ("" = all)
std::vector<ProfEvent> g_pev;
std::vector<hipEvent_t> g_pool;

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

template <class F>
int run(const char* name, hipStream_t s, F f) {
  hipEvent_t a = nullptr, b = nullptr;
  if (g_prof.load(std::memory_order_relaxed)) {
    std::lock_guard<std::mutex> lk(g_pm);
    if (g_pfilter.empty() || g_pfilter == name) {
      a = take_event();
      b = take_event();
      if (a) (void)hipEventRecord(a, s);
    }
  }
  hipError_t e = f();
  if (a && b) {
    (void)hipEventRecord(b, s);
    std::lock_guard<std::mutex> lk(g_pm);
    g_pev.push_back({name, a, b});
  }
  if (e != hipSuccess) return fail(K2_ERR_HIP, "%s: launch failed: %s", name, hipGetErrorString(e));
  return K2_OK;
}

#define K2_RUN(name, s, expr)                               \
  do {                                                      \
    int run_rc__ = run(name, s, [&]() -> hipError_t { return expr; }); \
    if (run_rc__ != K2_OK) return run_rc__;                 \
  } while (0)

// ---------------------------------------------------------------------------------------------
// Validation
// ---------------------------------------------------------------------------------------------
constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int check_block_cfg(const k2_block_cfg* c, bool rope) {
  if (!c) return fail(K2_ERR_NULL, "block config is NULL");
  if (c->dtype != K2_F32 && c->dtype != K2_BF16) return fail(K2_ERR_DTYPE, "unknown dtype %d", c->dtype);
  if (c->hidden <= 0 || c->num_heads <= 0 || c->num_kv_heads <= 0 || c->head_dim <= 0 || c->intermediate <= 0)
    return fail(K2_ERR_CONFIG, "block dimensions must be positive");
  if (c->hidden != c->num_heads * c->head_dim)
    return fail(K2_ERR_CONFIG, "hidden (%d) must equal num_heads * head_dim (%d * %d)", c->hidden, c->num_heads,
                c->head_dim);
  if (c->num_heads % c->num_kv_heads != 0) return fail(K2_ERR_CONFIG, "num_heads must be a multiple of num_kv_heads");
  const int G = c->num_heads / c->num_kv_heads;
  if (G != 1 && G != 2 && G != 4) return fail(K2_ERR_CONFIG, "num_heads / num_kv_heads must be 1, 2 or 4 (got %d)", G);
  if (c->head_dim != 64 && c->head_dim != 128) return fail(K2_ERR_CONFIG, "head_dim must be 64 or 128 (got %d)", c->head_dim);
  if (c->hidden % 8 != 0 || c->intermediate % 8 != 0)
    return fail(K2_ERR_CONFIG, "hidden and intermediate must be multiples of 8");
  if (!(c->eps >= 0.0f)) return fail(K2_ERR_CONFIG, "eps must be >= 0");
  if (rope) {
    const int* a = c->axes_dims;
    if (a[0] < 0 || a[1] < 0 || a[2] < 0 || a[0] % 2 || a[1] % 2 || a[2] % 2)
      return fail(K2_ERR_CONFIG, "axes_dims must be even and non-negative");
    if (a[0] + a[1] + a[2] != c->head_dim)
      return fail(K2_ERR_CONFIG, "sum(axes_dims) (%d) must equal head_dim (%d)", a[0] + a[1] + a[2], c->head_dim);
    if (!(c->rope_theta > 0.0f)) return fail(K2_ERR_CONFIG, "rope_theta must be > 0");
  }
  return K2_OK;
}

// Device pointers other than the workspace must be 16-byte aligned (NULL passes).
int check_align(const char* what, std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if ((uintptr_t)p & 15) return fail(K2_ERR_ALIGN, "%s: device pointer %p is not 16-byte aligned", what, p);
  return K2_OK;
}

int check_block_weights(const k2_block_weights* w) {
  if (!w) return fail(K2_ERR_NULL, "block weights are NULL");
  if (!w->to_q || !w->to_k || !w->to_v || !w->to_gate || !w->to_out || !w->ff_gate || !w->ff_up || !w->ff_down)
    return fail(K2_ERR_NULL, "a block projection weight is NULL");
  return check_align("block weights", {w->scale_shift_table, w->norm1_w, w->norm2_w, w->norm_q_w, w->norm_k_w, w->to_q,
                                       w->to_k, w->to_v, w->to_gate, w->to_out, w->ff_gate, w->ff_up, w->ff_down});
}

int check_sizes(int B, int T, int N) {
  if (B <= 0 || T < 0 || N < 0 || T + N <= 0) return fail(K2_ERR_SHAPE, "need B >= 1, T >= 0, N >= 0, T + N >= 1");
  if (B > 65535) return fail(K2_ERR_SHAPE, "B must be <= 65535");
  if ((long long)T + N > (1 << 24)) return fail(K2_ERR_SHAPE, "sequence too long");
  if (T > 16384) return fail(K2_ERR_SHAPE, "at most 16384 text tokens (got %d)", T);
  return K2_OK;
}

// The attention kernels reach one batch row's keys through one buffer descriptor (byte offsets below
// 0x7FFFFFF0: keys past it would read as zeros and take softmax mass) and index rows and V^T with
// 32-bit integers, so the sequence and the row count are bounded for the block's dims.
int check_extent(const k2_block_cfg* c, long long B, long long L) {
  const long long es = (long long)dt_size(c->dtype), nk = (long long)c->num_kv_heads * c->head_dim;
  const long long ldvt = L <= 32 ? 32 : (L + 63) / 64 * 64;
  if (B * L > INT_MAX) return fail(K2_ERR_SHAPE, "B * (T + N) = %lld rows exceeds 2^31 - 1", B * L);
  if (L * nk * es > 0x7FFFFFF0LL)
    return fail(K2_ERR_SHAPE, "sequence of %lld tokens too long: its keys (%lld bytes per batch row) exceed 2^31 - 16 bytes",
                L, L * nk * es);
  if (B * nk * ldvt > INT_MAX) return fail(K2_ERR_SHAPE, "B * kv columns * padded sequence exceeds 2^31 - 1");
  return K2_OK;
}

int check_ws(const void* ws, size_t have, size_t need) {
  if (need == 0) return K2_OK;
  if (!ws) return fail(K2_ERR_NULL, "workspace is NULL");
  if ((uintptr_t)ws % kAlign) return fail(K2_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (have < need) return fail(K2_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", have, need);
  return K2_OK;
}

// ---------------------------------------------------------------------------------------------
// Block workspace
// ---------------------------------------------------------------------------------------------
k2_block_workspace_layout block_layout(const k2_block_cfg* c, int B, int T, int N) {
  k2_block_workspace_layout l = {};
  const size_t es = dt_size(c->dtype);
  const size_t L = (size_t)T + N, M = (size_t)B * L;
  const size_t H = c->hidden, nq = (size_t)c->num_heads * c->head_dim, nk = (size_t)c->num_kv_heads * c->head_dim;
  // V^T rows: 64-key tiles for the tiled attention kernel, 32 key slots for short sequences
  l.ldvt = L <= 32 ? 32 : (int)((L + 63) / 64 * 64);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  l.x1 = take(M * H * es);
  l.q = take(M * nq * es);
  l.k = take(M * nk * es);
  l.vt = take((size_t)B * nk * l.ldvt * es);
  l.g = take(M * nq * es);
  l.og = take(M * nq * es);
  l.x2 = take(M * H * es);
  l.a = take(M * (size_t)c->intermediate * es);
  l.rope = take(2 * L * (size_t)(c->head_dim / 2) * sizeof(float));
  l.mod = take((size_t)B * 6 * H * sizeof(float));
  l.reach = take(L * sizeof(int32_t));
  l.total = off;
  return l;
}

char* at(void* base, size_t off) { return (char*)base + off; }

// One block forward; rope_cos/rope_sin precomputed by the caller when non-NULL.
// image_ids: (T + N) block ids of the block-causal attention, or NULL for attention over every key.
int block_run(const k2_block_cfg* c, const k2_block_weights* w, int B, int T, int N, const float* hin, float* hout,
              const float* temb, const float* pos, const uint8_t* mask, void* ws, const float* rope_cos,
              const float* rope_sin, hipStream_t s, const int32_t* image_ids = nullptr) {
  const int dt = c->dtype;
  const int H = c->hidden, hd = c->head_dim, nq = c->num_heads * hd, nk = c->num_kv_heads * hd, I = c->intermediate;
  const int L = T + N, M = B * L;
  const bool rope_inside = pos && !rope_cos;
  const k2_block_workspace_layout lay = block_layout(c, B, T, N);
  void* x1 = at(ws, lay.x1);
  void* q = at(ws, lay.q);
  void* k = at(ws, lay.k);
  void* vt = at(ws, lay.vt);
  void* g = at(ws, lay.g);
  void* og = at(ws, lay.og);
  void* x2 = at(ws, lay.x2);
  void* a = at(ws, lay.a);
  float* mod = (float*)at(ws, lay.mod);
  const bool modulated = w->scale_shift_table != nullptr;

  if (modulated) K2_RUN("modulation", s, modulation(temb, 6 * H, H, w->scale_shift_table, mod, B, 6, H, s));
  if (rope_inside) {
    rope_cos = (const float*)at(ws, lay.rope);
    rope_sin = rope_cos + (size_t)L * (hd / 2);
    K2_RUN("rope", s, rope_table(pos, L, c->axes_dims[0], c->axes_dims[1], c->axes_dims[2], c->rope_theta,
                                 (float*)rope_cos, (float*)rope_sin, s));
  }
  if (!pos) rope_cos = rope_sin = nullptr;

  ModnormArgs mn = {};
  mn.in = hin; mn.out = x1; mn.rows = M; mn.H = H;
  mn.rows_per_b = L; mn.in_rows_per_b = L; mn.in_row_off = 0;  // row r is batch r / L
  mn.w = w->norm1_w;
  mn.scale = modulated ? mod : nullptr;
  mn.shift = modulated ? mod + H : nullptr;
  mn.mod_stride = 6 * H;
  mn.eps = c->eps;
  K2_RUN("modnorm", s, modnorm(dt, mn, s));

  QkvgArgs qa = {};
  qa.wq = w->to_q; qa.wk = w->to_k; qa.wv = w->to_v; qa.wg = w->to_gate;
  qa.nq = nq; qa.nk = nk; qa.hd = hd; qa.L = L;
  qa.q = q; qa.k = k; qa.vt = vt; qa.g = g; qa.ldvt = lay.ldvt;
  qa.wnq = w->norm_q_w; qa.wnk = w->norm_k_w;
  qa.rope_cos = rope_cos; qa.rope_sin = rope_sin;
  qa.eps = c->eps;
  K2_RUN("gemm_qkvg", s, gemm_qkvg(dt, GemmA{x1, H, M, H}, qa, s));

  AttnArgs at_ = {};
  if (image_ids) {
    int* reach = (int*)at(ws, lay.reach);
    K2_RUN("block_reach", s, block_reach(image_ids, L, reach, s));
    at_.reach = reach;
  }
  at_.q = q; at_.k = k; at_.vt = vt; at_.g = g; at_.og = og; at_.mask = mask;
  at_.B = B; at_.L = L; at_.T = T; at_.nh = c->num_heads; at_.nkv = c->num_kv_heads; at_.hd = hd; at_.ldvt = lay.ldvt;
  K2_RUN("attention", s, attention(dt, at_, s));

  ResidArgs ro = {};
  ro.w = w->to_out; ro.N = H; ro.hin = hin; ro.hout = hout;
  ro.gate = modulated ? mod + 2 * H : nullptr; ro.gate_stride = 6 * H; ro.L = L;
  K2_RUN("gemm_out", s, gemm_resid(dt, GemmA{og, nq, M, nq}, ro, s));

  mn.in = hout; mn.out = x2; mn.w = w->norm2_w;
  mn.scale = modulated ? mod + 3 * H : nullptr;
  mn.shift = modulated ? mod + 4 * H : nullptr;
  K2_RUN("modnorm", s, modnorm(dt, mn, s));

  SwigluArgs sa = {};
  sa.wgate = w->ff_gate; sa.wup = w->ff_up; sa.I = I; sa.a = a;
  K2_RUN("gemm_swiglu", s, gemm_swiglu(dt, GemmA{x2, H, M, H}, sa, s));

  ResidArgs rd = {};
  rd.w = w->ff_down; rd.N = H; rd.hin = hout; rd.hout = hout;
  rd.gate = modulated ? mod + 5 * H : nullptr; rd.gate_stride = 6 * H; rd.L = L;
  K2_RUN("gemm_down", s, gemm_resid(dt, GemmA{a, I, M, I}, rd, s));
  return K2_OK;
}

int validate_block_call(const k2_block_cfg* cfg, const k2_block_weights* w, int B, int T, int N, const void* hin,
                        const void* hout, const float* temb, const float* pos, int pos_rows, int pos_cols) {
  int rc;
  if ((rc = check_block_cfg(cfg, pos != nullptr)) != K2_OK) return rc;
  if ((rc = check_block_weights(w)) != K2_OK) return rc;
  if ((rc = check_sizes(B, T, N)) != K2_OK) return rc;
  if ((rc = check_extent(cfg, B, (long long)T + N)) != K2_OK) return rc;
  if (!hin || !hout) return fail(K2_ERR_NULL, "hidden_in / hidden_out is NULL");
  if (w->scale_shift_table && !temb) return fail(K2_ERR_NULL, "temb is NULL but the block has a scale_shift_table");
  if (!w->scale_shift_table && temb) return fail(K2_ERR_CONFIG, "temb given for a block without scale_shift_table");
  if (pos && (pos_rows != T + N || pos_cols != 3))
    return fail(K2_ERR_SHAPE, "position_ids must be (T + N, 3) = (%d, 3), got (%d, %d)", T + N, pos_rows, pos_cols);
  return check_align("hidden_in / hidden_out / temb", {hin, hout, temb});
}

// ---------------------------------------------------------------------------------------------
// Time path
// ---------------------------------------------------------------------------------------------
struct TimeLayout {
  size_t emb, h1, ge, e, total;
};
TimeLayout time_layout(const k2_time_cfg* c, int B) {
  TimeLayout l = {};
  const size_t es = dt_size(c->dtype);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  l.emb = take((size_t)B * c->timestep_embed_dim * es);
  l.h1 = take((size_t)B * c->hidden * es);
  l.ge = take((size_t)B * c->hidden * es);
  l.e = take((size_t)B * c->hidden * sizeof(float));
  l.total = off;
  return l;
}

int check_time(const k2_time_cfg* c, const k2_time_weights* w, int B) {
  if (!c) return fail(K2_ERR_NULL, "time config is NULL");
  if (!w) return fail(K2_ERR_NULL, "time weights are NULL");
  if (c->dtype != K2_F32 && c->dtype != K2_BF16) return fail(K2_ERR_DTYPE, "unknown dtype %d", c->dtype);
  if (c->hidden <= 0 || c->hidden % 8) return fail(K2_ERR_CONFIG, "time hidden must be a positive multiple of 8");
  if (c->timestep_embed_dim <= 0 || c->timestep_embed_dim % 8)
    return fail(K2_ERR_CONFIG, "timestep_embed_dim must be a positive multiple of 8");
  if (!w->lin1_w || !w->lin2_w || !w->mod_w) return fail(K2_ERR_NULL, "a time-path weight is NULL");
  if (B <= 0) return fail(K2_ERR_SHAPE, "B must be >= 1");
  return check_align("time-path weights", {w->lin1_w, w->lin1_b, w->lin2_w, w->lin2_b, w->mod_w, w->mod_b});
}

int time_run(const k2_time_cfg* c, const k2_time_weights* w, int B, const float* t, float* temb, float* emb_out,
             void* ws, hipStream_t s) {
  const int dt = c->dtype, H = c->hidden, D = c->timestep_embed_dim;
  const TimeLayout l = time_layout(c, B);
  void* emb = at(ws, l.emb);
  void* h1 = at(ws, l.h1);
  void* ge = at(ws, l.ge);
  float* e = emb_out ? emb_out : (float*)at(ws, l.e);
  K2_RUN("time_embed", s, time_embed(dt, t, B, D, emb, s));
  PlainArgs p = {};
  p.w = w->lin1_w; p.N = H; p.bias = w->lin1_b; p.outt = h1; p.ldt = H; p.act = 1;
  p.rows_per_b = B; p.out_rows_per_b = B; p.out_row_off = 0;
  K2_RUN("gemm_plain", s, gemm_plain(dt, GemmA{emb, D, B, D}, p, s));
  p = PlainArgs{};
  p.w = w->lin2_w; p.N = H; p.bias = w->lin2_b; p.outf = e; p.ldf = H; p.outt = ge; p.ldt = H; p.act = 1;
  p.rows_per_b = B; p.out_rows_per_b = B; p.out_row_off = 0;
  K2_RUN("gemm_plain", s, gemm_plain(dt, GemmA{h1, H, B, H}, p, s));
  p = PlainArgs{};
  p.w = w->mod_w; p.N = 6 * H; p.bias = w->mod_b; p.outf = temb; p.ldf = 6 * H;
  p.rows_per_b = B; p.out_rows_per_b = B; p.out_row_off = 0;
  K2_RUN("gemm_plain", s, gemm_plain(dt, GemmA{ge, H, B, H}, p, s));
  return K2_OK;
}

// ---------------------------------------------------------------------------------------------
// Text fusion
// ---------------------------------------------------------------------------------------------
struct TextLayout {
  size_t xres, block, total;
  size_t block_bytes;
};
TextLayout text_layout(const k2_text_cfg* c, int B, int T) {
  TextLayout l = {};
  const size_t D = c->block.hidden;
  size_t off = 0;
  l.xres = off;
  off = align_up(off + (size_t)B * T * c->num_layers * D * sizeof(float));
  const size_t lw = block_layout(&c->block, B * T, 0, c->num_layers).total;
  const size_t rf = block_layout(&c->block, B, T, 0).total;
  l.block_bytes = lw > rf ? lw : rf;
  l.block = off;
  off = align_up(off + l.block_bytes);
  l.total = off;
  return l;
}

int check_text(const k2_text_cfg* c, const k2_text_weights* w, int B, int T) {
  if (!c) return fail(K2_ERR_NULL, "text config is NULL");
  int rc;
  if ((rc = check_block_cfg(&c->block, false)) != K2_OK) return rc;
  if (c->num_layers <= 0 || c->num_layerwise_blocks < 0 || c->num_refiner_blocks < 0)
    return fail(K2_ERR_CONFIG, "text fusion layer / block counts invalid");
  if (!w) return fail(K2_ERR_NULL, "text weights are NULL");
  if (!w->compress_w) return fail(K2_ERR_NULL, "compress_w is NULL");
  if (c->num_layerwise_blocks && !w->layerwise) return fail(K2_ERR_NULL, "layerwise block weights are NULL");
  if (c->num_refiner_blocks && !w->refiner) return fail(K2_ERR_NULL, "refiner block weights are NULL");
  for (int i = 0; i < c->num_layerwise_blocks; ++i) {
    if ((rc = check_block_weights(&w->layerwise[i])) != K2_OK) return rc;
    if (w->layerwise[i].scale_shift_table) return fail(K2_ERR_CONFIG, "text-fusion blocks take no modulation table");
  }
  for (int i = 0; i < c->num_refiner_blocks; ++i) {
    if ((rc = check_block_weights(&w->refiner[i])) != K2_OK) return rc;
    if (w->refiner[i].scale_shift_table) return fail(K2_ERR_CONFIG, "text-fusion blocks take no modulation table");
  }
  if (B <= 0 || T <= 0) return fail(K2_ERR_SHAPE, "text fusion needs B >= 1 and T >= 1");
  if ((long long)B * T > 65535) return fail(K2_ERR_SHAPE, "B * T must be <= 65535");
  if (T > 16384) return fail(K2_ERR_SHAPE, "at most 16384 text tokens (got %d)", T);
  if ((rc = check_extent(&c->block, (long long)B * T, c->num_layers)) != K2_OK) return rc;
  if ((rc = check_extent(&c->block, B, T)) != K2_OK) return rc;
  return K2_OK;
}

int text_run(const k2_text_cfg* c, const k2_text_weights* w, int B, int T, const void* enc, const uint8_t* mask,
             float* out, void* ws, hipStream_t s) {
  const TextLayout l = text_layout(c, B, T);
  const int D = c->block.hidden, NL = c->num_layers;
  float* xres = (float*)at(ws, l.xres);
  void* bws = at(ws, l.block);
  K2_RUN("convert", s, to_f32(c->block.dtype, enc, xres, (size_t)B * T * NL * D, s));
  for (int i = 0; i < c->num_layerwise_blocks; ++i) {
    int rc = block_run(&c->block, &w->layerwise[i], B * T, 0, NL, xres, xres, nullptr, nullptr, nullptr, bws, nullptr,
                       nullptr, s);
    if (rc != K2_OK) return rc;
  }
  K2_RUN("layer_compress", s, layer_compress(xres, w->compress_w, out, B * T, NL, D, s));
  for (int i = 0; i < c->num_refiner_blocks; ++i) {
    int rc = block_run(&c->block, &w->refiner[i], B, T, 0, out, out, nullptr, nullptr, mask, bws, nullptr, nullptr, s);
    if (rc != K2_OK) return rc;
  }
  return K2_OK;
}

// ---------------------------------------------------------------------------------------------
// Backbone
// ---------------------------------------------------------------------------------------------
struct ModelLayout {
  size_t temb, e, time, txt, txt_t, text, h, rope, block, fmod, xf, total;
};
// text: whether the call runs the text path itself (false: the caller passes its cached output)
ModelLayout model_layout(const k2_model_cfg* c, int B, int T, int N, bool text = true) {
  ModelLayout l = {};
  const size_t es = dt_size(c->block.dtype);
  const size_t H = c->block.hidden, L = (size_t)T + N, Dt = c->text.block.hidden;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  k2_time_cfg tc = {c->block.hidden, c->timestep_embed_dim, c->block.dtype};
  l.temb = take((size_t)B * 6 * H * sizeof(float));
  l.e = take((size_t)B * H * sizeof(float));
  l.time = take(time_layout(&tc, B).total);
  const size_t Tt = text ? (size_t)T : 0;
  l.txt = take((size_t)B * Tt * Dt * sizeof(float));
  l.txt_t = take((size_t)B * Tt * Dt * es);
  l.text = take(Tt > 0 ? text_layout(&c->text, B, T).total : 0);
  l.h = take((size_t)B * L * H * sizeof(float));
  l.rope = take(2 * L * (size_t)(c->block.head_dim / 2) * sizeof(float));
  l.block = take(block_layout(&c->block, B, T, N).total);
  l.fmod = take((size_t)B * 2 * H * sizeof(float));
  l.xf = take((size_t)B * N * H * es);
  l.total = off;
  return l;
}

int check_model(const k2_model_cfg* c, const k2_model_weights* w, int B, int T, int N, bool text = true) {
  if (!c) return fail(K2_ERR_NULL, "model config is NULL");
  int rc;
  if ((rc = check_block_cfg(&c->block, true)) != K2_OK) return rc;
  if (c->text.block.dtype != c->block.dtype) return fail(K2_ERR_DTYPE, "text and block dtypes differ");
  if (c->num_layers < 0 || c->in_channels <= 0 || c->in_channels % 8 || c->timestep_embed_dim <= 0 ||
      c->timestep_embed_dim % 8)
    return fail(K2_ERR_CONFIG, "num_layers >= 0, in_channels and timestep_embed_dim positive multiples of 8");
  if (c->text.block.hidden % 8) return fail(K2_ERR_CONFIG, "text hidden must be a multiple of 8");
  if (!w) return fail(K2_ERR_NULL, "model weights are NULL");
  if (!w->img_in_w || (text && !w->txt_in_w) || !w->final_w || !w->final_table)
    return fail(K2_ERR_NULL, "img_in / txt_in / final weights are NULL");
  if ((rc = check_align("img_in / txt_in / final weights", {w->img_in_w, w->img_in_b, w->txt_in_w, w->txt_in_b,
                                                            w->final_w, w->final_b, w->final_norm_w,
                                                            w->final_table})) != K2_OK)
    return rc;
  if (c->num_layers && !w->blocks) return fail(K2_ERR_NULL, "block weights are NULL");
  for (int i = 0; i < c->num_layers; ++i) {
    if ((rc = check_block_weights(&w->blocks[i])) != K2_OK) return rc;
    if (!w->blocks[i].scale_shift_table) return fail(K2_ERR_NULL, "block %d has no scale_shift_table", i);
  }
  k2_time_cfg tc = {c->block.hidden, c->timestep_embed_dim, c->block.dtype};
  if ((rc = check_time(&tc, &w->time, B)) != K2_OK) return rc;
  if ((rc = check_sizes(B, T, N)) != K2_OK) return rc;
  if ((rc = check_extent(&c->block, B, (long long)T + N)) != K2_OK) return rc;
  if (N <= 0) return fail(K2_ERR_SHAPE, "the backbone needs N >= 1 image tokens");
  if (text && T > 0 && (rc = check_text(&c->text, &w->text, B, T)) != K2_OK) return rc;
  return K2_OK;
}

// txt_in(text_fusion(enc)) into rows [0, T) of every batch row of out (out_rows_per_b rows per batch
// row, width hidden, float32). ws: text_embed_layout(c, B, T).total bytes.
struct TextEmbedLayout {
  size_t txt, txt_t, text, total;
};
TextEmbedLayout text_embed_layout(const k2_model_cfg* c, int B, int T) {
  TextEmbedLayout l = {};
  const size_t es = dt_size(c->block.dtype), Dt = c->text.block.hidden;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  l.txt = take((size_t)B * T * Dt * sizeof(float));
  l.txt_t = take((size_t)B * T * Dt * es);
  l.text = take(T > 0 ? text_layout(&c->text, B, T).total : 0);
  l.total = off;
  return l;
}

int text_embed_run(const k2_model_cfg* cfg, const k2_model_weights* w, int B, int T, const void* enc,
                   const uint8_t* mask, float* out, int out_rows_per_b, void* ws, hipStream_t s) {
  if (T <= 0) return K2_OK;
  const TextEmbedLayout l = text_embed_layout(cfg, B, T);
  const int dt = cfg->block.dtype, H = cfg->block.hidden, Dt = cfg->text.block.hidden;
  float* txt = (float*)at(ws, l.txt);
  void* txt_t = at(ws, l.txt_t);
  int rc;
  if ((rc = text_run(&cfg->text, &w->text, B, T, enc, mask, txt, at(ws, l.text), s)) != K2_OK) return rc;
  K2_RUN("convert", s, from_f32(dt, txt, txt_t, (size_t)B * T * Dt, s));
  PlainArgs p = {};
  p.w = w->txt_in_w; p.N = H; p.bias = w->txt_in_b; p.outf = out; p.ldf = H;
  p.rows_per_b = T; p.out_rows_per_b = out_rows_per_b; p.out_row_off = 0;
  K2_RUN("gemm_plain", s, gemm_plain(dt, GemmA{txt_t, Dt, B * T, Dt}, p, s));
  return K2_OK;
}

// ---------------------------------------------------------------------------------------------
// Block backward: recompute the forward from the block input keeping what the chain rule needs,
// then the gradients step by step in reverse. Every matrix product is the forward's GEMM with a
// plain epilogue, fed K-contiguous operands by transposes.
// ---------------------------------------------------------------------------------------------
constexpr int kBwdRows = 16;  // rows per partial-sum chunk of the column reductions

struct BwdLayout {
  // recompute
  size_t mod, rope, x1, qraw, kraw, q, k, vt, vrow, kt, g, o, og, lse, y, h1, x2, gt, u, a, z;
  // backward
  size_t dh1, dz, dzT, aT, da, dgu, dguT, x2T, dx2, dy, dyT, ogT, dog, dO, dOT, qT, delta, dq, dk, dkv_part, dqkvg,
      dqkvgT, x1T, dx1, wT, dmod, dwqkvg;
  size_t p_qg, p_pg, p_w2, p_qs, p_qt, p_w1, p_ps, p_pt, p_wq, p_wk;
  int ldvt, Mp, ncb, qk_blocks;
  size_t total;
};

BwdLayout bwd_layout(const k2_block_cfg* c, int B, int T, int N) {
  BwdLayout l = {};
  const size_t es = dt_size(c->dtype), f4 = sizeof(float);
  const size_t L = (size_t)T + N, M = (size_t)B * L;
  const size_t H = c->hidden, I = c->intermediate, hd = c->head_dim;
  const size_t nq = (size_t)c->num_heads * hd, nk = (size_t)c->num_kv_heads * hd, nall = 2 * nq + 2 * nk;
  l.ldvt = L <= 32 ? 32 : (int)((L + 63) / 64 * 64);
  l.Mp = (int)((M + 63) / 64 * 64);
  l.ncb = (int)((L + kBwdRows - 1) / kBwdRows);
  l.qk_blocks = 1024;
  const size_t Mp = l.Mp, chunks = (size_t)B * l.ncb;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  l.mod = take((size_t)B * 6 * H * f4);
  l.rope = take(2 * L * (hd / 2) * f4);
  l.x1 = take(M * H * es);
  l.qraw = take(M * nq * f4);
  l.kraw = take(M * nk * f4);
  l.q = take(M * nq * es);
  l.k = take(M * nk * es);
  l.vt = take((size_t)B * nk * l.ldvt * es);
  l.vrow = take(M * nk * es);
  l.kt = take((size_t)B * nk * l.ldvt * es);
  l.g = take(M * nq * es);
  l.o = take(M * nq * es);
  l.og = take(M * nq * es);
  l.lse = take((size_t)B * c->num_heads * L * f4);
  l.y = take(M * H * f4);
  l.h1 = take(M * H * f4);
  l.x2 = take(M * H * es);
  l.gt = take(M * I * f4);
  l.u = take(M * I * f4);
  l.a = take(M * I * es);
  l.z = take(M * H * f4);
  l.dh1 = take(M * H * f4);
  l.dz = take(M * H * es);
  l.dzT = take(H * Mp * es);
  l.aT = take(I * Mp * es);
  l.da = take(M * I * f4);
  l.dgu = take(M * 2 * I * es);
  l.dguT = take(2 * I * Mp * es);
  l.x2T = take(H * Mp * es);
  l.dx2 = take(M * H * f4);
  l.dy = take(M * H * es);
  l.dyT = take(H * Mp * es);
  l.ogT = take(nq * Mp * es);
  l.dog = take(M * nq * f4);
  l.dO = take(M * nq * es);
  l.dOT = take((size_t)B * nq * l.ldvt * es);
  l.qT = take((size_t)B * nq * l.ldvt * es);
  l.delta = take((size_t)B * c->num_heads * L * f4);
  l.dq = take(M * nq * f4);
  l.dk = take(M * nk * f4);
  l.dkv_part = take(4 * M * nk * f4);  // dK / dV partial sums of a split dK/dV pass
  l.dqkvg = take(M * nall * es);
  l.dqkvgT = take(nall * Mp * es);
  l.x1T = take(H * Mp * es);
  l.dx1 = take(M * H * f4);
  l.wT = take(std::max({I * H, H * 2 * I, nq * H, H * nall}) * es);
  l.dmod = take((size_t)B * 6 * H * f4);
  l.dwqkvg = take(nall * H * f4);  // [dWq; dWk; dWv; dWg] before they are copied out
  l.p_qg = take(chunks * H * f4);
  l.p_pg = take(chunks * H * f4);
  l.p_w2 = take(chunks * H * f4);
  l.p_qs = take(chunks * H * f4);
  l.p_qt = take(chunks * H * f4);
  l.p_w1 = take(chunks * H * f4);
  l.p_ps = take(chunks * H * f4);
  l.p_pt = take(chunks * H * f4);
  l.p_wq = take((size_t)l.qk_blocks * hd * f4);
  l.p_wk = take((size_t)l.qk_blocks * hd * f4);
  l.total = off;
  return l;
}

// dst (C x Rpad, row stride ldd) = transpose of src (R x C, row stride lds), zeros in rows past R
hipError_t transpose2d(int dt, const void* src, int R, int C, int lds, void* dst, int Rpad, int ldd, hipStream_t s) {
  TransposeArgs t = {};
  t.src = src; t.dst = dst; t.R = R; t.C = C; t.Rpad = Rpad; t.lds = lds; t.ldd = ldd; t.Z = 1; t.zdiv = 1;
  return transpose(dt, t, s);
}

// per (batch, head): (B, L, heads, hd) row-major -> (B, heads, hd, ldt)
hipError_t transpose_heads(int dt, const void* src, int B, int L, int heads, int hd, void* dst, int ldt, hipStream_t s) {
  TransposeArgs t = {};
  t.src = src; t.dst = dst; t.R = L; t.C = hd; t.Rpad = ldt; t.lds = heads * hd; t.ldd = ldt;
  t.Z = B * heads; t.zdiv = heads;
  t.sz0 = (size_t)L * heads * hd; t.sz1 = hd;
  t.dz0 = (size_t)heads * hd * ldt; t.dz1 = (size_t)hd * ldt;
  return transpose(dt, t, s);
}

// C (rows x N) float32 = A (rows x K) * Bw (N x K)^T, both K-contiguous with row strides lda and K
hipError_t gemm_f32out(int dt, const void* A, int lda, int rows, int K, const void* Bw, int N, float* C, int ldc,
                       hipStream_t s) {
  PlainArgs p = {};
  p.w = Bw; p.N = N; p.outf = C; p.ldf = ldc;
  p.rows_per_b = rows; p.out_rows_per_b = rows; p.out_row_off = 0;
  return gemm_plain(dt, GemmA{A, lda, rows, K}, p, s);
}

int block_backward_run(const k2_block_cfg* c, const k2_block_weights* w, int B, int T, int N, const float* hin,
                       const float* temb, const float* pos, const uint8_t* mask, const float* dh2, float* dh_in,
                       float* dtemb, const k2_block_grads* gr, void* ws, hipStream_t s) {
  const int dt = c->dtype;
  const int H = c->hidden, hd = c->head_dim, nh = c->num_heads, nkv = c->num_kv_heads, I = c->intermediate;
  const int nq = nh * hd, nk = nkv * hd, nall = 2 * nq + 2 * nk;
  const int L = T + N, M = B * L;
  const BwdLayout l = bwd_layout(c, B, T, N);
  const int Mp = l.Mp, ldt = l.ldvt;
  const bool modulated = w->scale_shift_table != nullptr;
  auto P = [&](size_t off) { return at(ws, off); };
  float* mod = (float*)P(l.mod);
  const float* ps = modulated ? mod : nullptr;
  const float* pt = modulated ? mod + H : nullptr;
  const float* pg = modulated ? mod + 2 * H : nullptr;
  const float* qs = modulated ? mod + 3 * H : nullptr;
  const float* qt = modulated ? mod + 4 * H : nullptr;
  const float* qg = modulated ? mod + 5 * H : nullptr;
  const int ms = 6 * H;

  // ---- recompute the forward from hin
  if (modulated) K2_RUN("modulation", s, modulation(temb, 6 * H, H, w->scale_shift_table, mod, B, 6, H, s));
  float* rc = nullptr;
  float* rsn = nullptr;
  if (pos) {
    rc = (float*)P(l.rope);
    rsn = rc + (size_t)L * (hd / 2);
    K2_RUN("rope", s, rope_table(pos, L, c->axes_dims[0], c->axes_dims[1], c->axes_dims[2], c->rope_theta, rc, rsn, s));
  }
  ModnormArgs mn = {};
  mn.in = hin; mn.out = P(l.x1); mn.rows = M; mn.H = H;
  mn.rows_per_b = L; mn.in_rows_per_b = L; mn.in_row_off = 0;
  mn.w = w->norm1_w; mn.scale = ps; mn.shift = pt; mn.mod_stride = ms; mn.eps = c->eps;
  K2_RUN("modnorm", s, modnorm(dt, mn, s));
  QkvgArgs qa = {};
  qa.wq = w->to_q; qa.wk = w->to_k; qa.wv = w->to_v; qa.wg = w->to_gate;
  qa.nq = nq; qa.nk = nk; qa.hd = hd; qa.L = L;
  qa.q = P(l.q); qa.k = P(l.k); qa.vt = P(l.vt); qa.g = P(l.g); qa.ldvt = ldt;
  qa.wnq = w->norm_q_w; qa.wnk = w->norm_k_w; qa.rope_cos = rc; qa.rope_sin = rsn; qa.eps = c->eps;
  qa.qraw = (float*)P(l.qraw); qa.kraw = (float*)P(l.kraw); qa.vrow = P(l.vrow); qa.kt = P(l.kt);
  K2_RUN("gemm_qkvg", s, gemm_qkvg(dt, GemmA{P(l.x1), H, M, H}, qa, s));
  AttnArgs aa = {};
  aa.q = P(l.q); aa.k = P(l.k); aa.vt = P(l.vt); aa.g = P(l.g); aa.og = P(l.og); aa.mask = mask;
  aa.B = B; aa.L = L; aa.T = T; aa.nh = nh; aa.nkv = nkv; aa.hd = hd; aa.ldvt = ldt;
  aa.o_pre = P(l.o); aa.lse = (float*)P(l.lse);
  K2_RUN("attention", s, attention(dt, aa, s));
  float* y = (float*)P(l.y);
  float* h1 = (float*)P(l.h1);
  K2_RUN("gemm_plain", s, gemm_f32out(dt, P(l.og), nq, M, nq, w->to_out, H, y, H, s));
  K2_RUN("gated_add", s, gated_add(hin, y, pg, ms, L, M, H, h1, s));
  mn.in = h1; mn.out = P(l.x2); mn.w = w->norm2_w; mn.scale = qs; mn.shift = qt;
  K2_RUN("modnorm", s, modnorm(dt, mn, s));
  SwigluArgs sa = {};
  sa.wgate = w->ff_gate; sa.wup = w->ff_up; sa.I = I; sa.a = P(l.a);
  sa.gsave = (float*)P(l.gt); sa.usave = (float*)P(l.u);
  K2_RUN("gemm_swiglu", s, gemm_swiglu(dt, GemmA{P(l.x2), H, M, H}, sa, s));
  float* z = (float*)P(l.z);
  K2_RUN("gemm_plain", s, gemm_f32out(dt, P(l.a), I, M, I, w->ff_down, H, z, H, s));

  // ---- backward, in reverse
  GatedGradArgs gg = {};
  gg.dh = dh2; gg.br = modulated ? z : nullptr; gg.gate = qg; gg.gate_stride = ms; gg.out = P(l.dz);
  gg.part = modulated ? (float*)P(l.p_qg) : nullptr;
  gg.B = B; gg.L = L; gg.H = H; gg.RC = kBwdRows; gg.ncb = l.ncb;
  K2_RUN("gated_grad", s, gated_grad(dt, gg, s));  // dz = qg dh2; dqg partials
  if (gr->ff_down) {  // dWd = dz^T a
    K2_RUN("transpose", s, transpose2d(dt, P(l.dz), M, H, H, P(l.dzT), Mp, Mp, s));
    K2_RUN("transpose", s, transpose2d(dt, P(l.a), M, I, I, P(l.aT), Mp, Mp, s));
    K2_RUN("gemm_plain", s, gemm_f32out(dt, P(l.dzT), Mp, H, Mp, P(l.aT), I, gr->ff_down, I, s));
  }
  // da = dz Wd
  K2_RUN("transpose", s, transpose2d(dt, w->ff_down, H, I, I, P(l.wT), H, H, s));
  K2_RUN("gemm_plain", s, gemm_f32out(dt, P(l.dz), H, M, H, P(l.wT), I, (float*)P(l.da), I, s));
  K2_RUN("swiglu_bwd", s, swiglu_bwd(dt, (float*)P(l.da), (float*)P(l.gt), (float*)P(l.u), M, I, P(l.dgu), s));
  if (gr->ff_gate || gr->ff_up) {  // [dWgate; dWup] = [dgt du]^T x2
    K2_RUN("transpose", s, transpose2d(dt, P(l.dgu), M, 2 * I, 2 * I, P(l.dguT), Mp, Mp, s));
    K2_RUN("transpose", s, transpose2d(dt, P(l.x2), M, H, H, P(l.x2T), Mp, Mp, s));
    if (gr->ff_gate)
      K2_RUN("gemm_plain", s, gemm_f32out(dt, P(l.dguT), Mp, I, Mp, P(l.x2T), H, gr->ff_gate, H, s));
    if (gr->ff_up)
      K2_RUN("gemm_plain", s, gemm_f32out(dt, at(P(l.dguT), (size_t)I * Mp * dt_size(dt)), Mp, I, Mp, P(l.x2T), H,
                                          gr->ff_up, H, s));
  }
  // dx2 = dgt Wgate + du Wup, as two products over K = I: the second adds onto the first through
  // the residual epilogue (no gate). One product over K = 2I read 403 MB of weights, more than the
  // last-level cache holds (3.55 ms); each half's 201 MB stays there.
  void* const wTu = at(P(l.wT), (size_t)H * I * dt_size(dt));
  K2_RUN("transpose", s, transpose2d(dt, w->ff_gate, I, H, H, P(l.wT), I, I, s));
  K2_RUN("transpose", s, transpose2d(dt, w->ff_up, I, H, H, wTu, I, I, s));
  K2_RUN("gemm_plain", s, gemm_f32out(dt, P(l.dgu), 2 * I, M, I, P(l.wT), H, (float*)P(l.dx2), H, s));
  {
    ResidArgs ra = {};
    ra.w = wTu; ra.N = H; ra.hin = (float*)P(l.dx2); ra.hout = (float*)P(l.dx2); ra.gate = nullptr;
    ra.gate_stride = 0; ra.L = M;
    K2_RUN("gemm_plain", s, gemm_resid(dt, GemmA{at(P(l.dgu), (size_t)I * dt_size(dt)), 2 * I, M, I}, ra, s));
  }
  // norm 2: dh1 = dh2 + its input gradient; partials for norm2_w, dqs, dqt
  NormBwdArgs nb = {};
  nb.x = h1; nb.dout = (float*)P(l.dx2); nb.dres = dh2; nb.dx = (float*)P(l.dh1);
  nb.w = w->norm2_w; nb.scale = qs; nb.mod_stride = ms;
  nb.pw = (float*)P(l.p_w2); nb.psc = (float*)P(l.p_qs); nb.psh = (float*)P(l.p_qt);
  nb.B = B; nb.L = L; nb.H = H; nb.RC = kBwdRows; nb.ncb = l.ncb; nb.eps = c->eps;
  K2_RUN("norm_bwd", s, norm_bwd(nb, s));
  float* dh1 = (float*)P(l.dh1);
  gg = GatedGradArgs{};
  gg.dh = dh1; gg.br = modulated ? y : nullptr; gg.gate = pg; gg.gate_stride = ms; gg.out = P(l.dy);
  gg.part = modulated ? (float*)P(l.p_pg) : nullptr;
  gg.B = B; gg.L = L; gg.H = H; gg.RC = kBwdRows; gg.ncb = l.ncb;
  K2_RUN("gated_grad", s, gated_grad(dt, gg, s));  // dy = pg dh1; dpg partials
  if (gr->to_out) {  // dWo = dy^T og
    K2_RUN("transpose", s, transpose2d(dt, P(l.dy), M, H, H, P(l.dyT), Mp, Mp, s));
    K2_RUN("transpose", s, transpose2d(dt, P(l.og), M, nq, nq, P(l.ogT), Mp, Mp, s));
    K2_RUN("gemm_plain", s, gemm_f32out(dt, P(l.dyT), Mp, H, Mp, P(l.ogT), nq, gr->to_out, nq, s));
  }
  // dog = dy Wo
  K2_RUN("transpose", s, transpose2d(dt, w->to_out, H, nq, nq, P(l.wT), H, H, s));
  K2_RUN("gemm_plain", s, gemm_f32out(dt, P(l.dy), H, M, H, P(l.wT), nq, (float*)P(l.dog), nq, s));
  // output gate: dO, dgraw (into the gate columns of dqkvg), Delta
  GateBwdArgs gb = {};
  gb.dog = (float*)P(l.dog); gb.g = P(l.g); gb.o = P(l.o); gb.dout = P(l.dO);
  gb.dg = at(P(l.dqkvg), (size_t)(nq + 2 * nk) * dt_size(dt)); gb.ldg = nall;
  gb.delta = (float*)P(l.delta); gb.M = M; gb.L = L; gb.nh = nh; gb.nq = nq; gb.hd = hd;
  K2_RUN("gate_bwd", s, gate_bwd(dt, gb, s));
  // attention
  K2_RUN("transpose", s, transpose_heads(dt, P(l.q), B, L, nh, hd, P(l.qT), ldt, s));
  K2_RUN("transpose", s, transpose_heads(dt, P(l.dO), B, L, nh, hd, P(l.dOT), ldt, s));
  AttnBwdArgs ab = {};
  ab.q = P(l.q); ab.k = P(l.k); ab.v = P(l.vrow); ab.qt = P(l.qT); ab.kt = P(l.kt); ab.dot = P(l.dOT);
  ab.dout = P(l.dO); ab.lse = (float*)P(l.lse); ab.delta = (float*)P(l.delta); ab.mask = mask;
  ab.dq = (float*)P(l.dq); ab.lddq = nq; ab.dk = (float*)P(l.dk); ab.lddk = nk;
  ab.dv = at(P(l.dqkvg), (size_t)(nq + nk) * dt_size(dt)); ab.lddv = nall;
  ab.dkv_part = (float*)P(l.dkv_part);
  ab.B = B; ab.L = L; ab.T = T; ab.nh = nh; ab.nkv = nkv; ab.hd = hd; ab.ldt = ldt;
  K2_RUN("attention_bwd", s, attention_backward(dt, ab, s));
  // q / k: RoPE transpose + head norm backward into the q and k columns of dqkvg
  QkNormBwdArgs qn = {};
  qn.dr = (float*)P(l.dq); qn.lddr = nq; qn.x = (float*)P(l.qraw); qn.ldx = nq; qn.rc = rc; qn.rs = rsn;
  qn.w = w->norm_q_w; qn.dx = P(l.dqkvg); qn.lddx = nall; qn.part = (float*)P(l.p_wq);
  qn.M = M; qn.L = L; qn.heads = nh; qn.hd = hd; qn.eps = c->eps;
  K2_RUN("qknorm_bwd", s, qknorm_bwd(dt, qn, l.qk_blocks, s));
  qn.dr = (float*)P(l.dk); qn.lddr = nk; qn.x = (float*)P(l.kraw); qn.ldx = nk; qn.w = w->norm_k_w;
  qn.dx = at(P(l.dqkvg), (size_t)nq * dt_size(dt)); qn.part = (float*)P(l.p_wk); qn.heads = nkv;
  K2_RUN("qknorm_bwd", s, qknorm_bwd(dt, qn, l.qk_blocks, s));
  // projection weights: [dWq; dWk; dWv; dWg] = dqkvg^T x1
  if (gr->to_q || gr->to_k || gr->to_v || gr->to_gate) {
    K2_RUN("transpose", s, transpose2d(dt, P(l.dqkvg), M, nall, nall, P(l.dqkvgT), Mp, Mp, s));
    K2_RUN("transpose", s, transpose2d(dt, P(l.x1), M, H, H, P(l.x1T), Mp, Mp, s));
    // one product for the four weights (their 1536-row k and v parts alone filled 144 of the 256
    // compute units), then each requested part copied out
    float* outs[4] = {gr->to_q, gr->to_k, gr->to_v, gr->to_gate};
    const int start[4] = {0, nq, nq + nk, nq + 2 * nk}, rows[4] = {nq, nk, nk, nq};
    float* const dwall = (float*)P(l.dwqkvg);
    K2_RUN("gemm_plain", s, gemm_f32out(dt, P(l.dqkvgT), Mp, nall, Mp, P(l.x1T), H, dwall, H, s));
    for (int i = 0; i < 4; ++i)
      if (outs[i]) {
        const hipError_t e = hipMemcpyAsync(outs[i], dwall + (size_t)start[i] * H, (size_t)rows[i] * H * sizeof(float),
                                            hipMemcpyDeviceToDevice, s);
        if (e != hipSuccess) return fail(K2_ERR_HIP, "weight gradient copy: %s", hipGetErrorString(e));
      }
  }
  // dx1 = dqkvg [Wq; Wk; Wv; Wg]
  {
    const void* ws4[4] = {w->to_q, w->to_k, w->to_v, w->to_gate};
    const int start[4] = {0, nq, nq + nk, nq + 2 * nk}, rows[4] = {nq, nk, nk, nq};
    for (int i = 0; i < 4; ++i)
      K2_RUN("transpose", s, transpose2d(dt, ws4[i], rows[i], H, H, at(P(l.wT), (size_t)start[i] * dt_size(dt)),
                                         rows[i], nall, s));
  }
  K2_RUN("gemm_plain", s, gemm_f32out(dt, P(l.dqkvg), nall, M, nall, P(l.wT), H, (float*)P(l.dx1), H, s));
  // norm 1: dh = dh1 + its input gradient; partials for norm1_w, dps, dpt
  nb = NormBwdArgs{};
  nb.x = hin; nb.dout = (float*)P(l.dx1); nb.dres = dh1; nb.dx = dh_in;
  nb.w = w->norm1_w; nb.scale = ps; nb.mod_stride = ms;
  nb.pw = (float*)P(l.p_w1); nb.psc = (float*)P(l.p_ps); nb.psh = (float*)P(l.p_pt);
  nb.B = B; nb.L = L; nb.H = H; nb.RC = kBwdRows; nb.ncb = l.ncb; nb.eps = c->eps;
  K2_RUN("norm_bwd", s, norm_bwd(nb, s));

  // ---- reductions of the partial sums
  // (independent column sums in one launch; the table's gradient sums the temb gradient after it)
  const int chunks = B * l.ncb;
  ReduceJobs rj = {};
  auto add_job = [&](const float* part, int G, int nc, int ncols, int ldp, float* out, int ldo) {
    rj.job[rj.n++] = ReduceJob{part, out, G, nc, ncols, ldp, ldo};
  };
  if (gr->norm1_w) add_job((float*)P(l.p_w1), 1, chunks, H, H, gr->norm1_w, H);
  if (gr->norm2_w) add_job((float*)P(l.p_w2), 1, chunks, H, H, gr->norm2_w, H);
  if (gr->norm_q_w) add_job((float*)P(l.p_wq), 1, l.qk_blocks, hd, hd, gr->norm_q_w, hd);
  if (gr->norm_k_w) add_job((float*)P(l.p_wk), 1, l.qk_blocks, hd, hd, gr->norm_k_w, hd);
  float* dm = nullptr;
  if (modulated && (dtemb || gr->scale_shift_table)) {
    dm = dtemb ? dtemb : (float*)P(l.dmod);
    const size_t parts[6] = {l.p_ps, l.p_pt, l.p_pg, l.p_qs, l.p_qt, l.p_qg};  // the chunk order of the modulation
    for (int cc = 0; cc < 6; ++cc) add_job((float*)P(parts[cc]), B, l.ncb, H, H, dm + (size_t)cc * H, 6 * H);
  }
  K2_RUN("reduce_rows", s, reduce_rows_multi(rj, s));
  if (dm && gr->scale_shift_table)
    K2_RUN("reduce_rows", s, reduce_rows(dm, 1, B, 6 * H, 6 * H, gr->scale_shift_table, 6 * H, s));
  return K2_OK;
}

}  // namespace

// =================================================================================================
// Exported entry points
// =================================================================================================
extern "C" {

void k2_block_cfg_default(k2_block_cfg* c) {
  if (!c) return;
  c->hidden = 6144;
  c->num_heads = 48;
  c->num_kv_heads = 12;
  c->head_dim = 128;
  c->intermediate = 16384;
  c->axes_dims[0] = 32;
  c->axes_dims[1] = 48;
  c->axes_dims[2] = 48;
  c->rope_theta = 1000.0f;
  c->eps = 1e-5f;
  c->dtype = K2_BF16;
}

void k2_text_cfg_default(k2_text_cfg* c) {
  if (!c) return;
  k2_block_cfg_default(&c->block);
  c->block.hidden = 2560;
  c->block.num_heads = 20;
  c->block.num_kv_heads = 20;
  c->block.head_dim = 128;
  c->block.intermediate = 6912;
  c->block.axes_dims[0] = c->block.axes_dims[1] = c->block.axes_dims[2] = 0;
  c->num_layers = 12;
  c->num_layerwise_blocks = 2;
  c->num_refiner_blocks = 2;
}

void k2_model_cfg_default(k2_model_cfg* c) {
  if (!c) return;
  k2_block_cfg_default(&c->block);
  k2_text_cfg_default(&c->text);
  c->num_layers = 28;
  c->in_channels = 64;
  c->timestep_embed_dim = 256;
}

size_t k2_block_workspace_bytes(const k2_block_cfg* cfg, int B, int T, int N) {
  if (!cfg || B < 0 || T < 0 || N < 0) return 0;
  return block_layout(cfg, B, T, N).total;
}

int k2_block_workspace_layout_query(const k2_block_cfg* cfg, int B, int T, int N, k2_block_workspace_layout* out) {
  if (!cfg || !out) return fail(K2_ERR_NULL, "config or output is NULL");
  if (B < 0 || T < 0 || N < 0) return fail(K2_ERR_SHAPE, "negative size");
  *out = block_layout(cfg, B, T, N);
  return K2_OK;
}

int k2_block_forward(const k2_block_cfg* cfg, const k2_block_weights* w, int B, int T, int N, const float* hidden_in,
                     float* hidden_out, const float* temb, const float* position_ids, int pos_rows, int pos_cols,
                     const uint8_t* mask, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = validate_block_call(cfg, w, B, T, N, hidden_in, hidden_out, temb, position_ids, pos_rows, pos_cols);
  if (rc != K2_OK) return rc;
  if ((rc = check_ws(workspace, workspace_bytes, k2_block_workspace_bytes(cfg, B, T, N))) != K2_OK) return rc;
  g_err.clear();
  return block_run(cfg, w, B, T, N, hidden_in, hidden_out, temb, position_ids, mask, workspace, nullptr, nullptr,
                   (hipStream_t)stream);
}

int k2_block_forward_block_causal(const k2_block_cfg* cfg, const k2_block_weights* w, int B, int T, int N,
                                  const float* hidden_in, float* hidden_out, const float* temb,
                                  const float* position_ids, int pos_rows, int pos_cols, const uint8_t* mask,
                                  const int32_t* image_ids, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = validate_block_call(cfg, w, B, T, N, hidden_in, hidden_out, temb, position_ids, pos_rows, pos_cols);
  if (rc != K2_OK) return rc;
  if (!image_ids) return fail(K2_ERR_NULL, "image_ids is NULL");
  if ((uintptr_t)image_ids % sizeof(int32_t)) return fail(K2_ERR_ALIGN, "image_ids must be 4-byte aligned");
  if ((rc = check_ws(workspace, workspace_bytes, k2_block_workspace_bytes(cfg, B, T, N))) != K2_OK) return rc;
  g_err.clear();
  return block_run(cfg, w, B, T, N, hidden_in, hidden_out, temb, position_ids, mask, workspace, nullptr, nullptr,
                   (hipStream_t)stream, image_ids);
}

// ---------------------------------------------------------------------------------------------
// Block forward without a caller workspace: the workspace is a file-scope device array. Host code
// never names the array itself (in host code its name is a stand-in, not a device address); its
// address on each device is taken once with hipGetSymbolAddress and kept per device.
// ---------------------------------------------------------------------------------------------
constexpr size_t kStaticScratchBytes = size_t(128) << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

std::mutex g_scratch_m;
std::vector<void*> g_scratch_ptr;  // device index -> address of `scratch` on that device

// Address of the static scratch on the current device (looked up on the first call per device).
int static_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0) return fail(K2_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lk(g_scratch_m);
  if ((size_t)dev >= g_scratch_ptr.size()) g_scratch_ptr.resize(dev + 1, nullptr);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(K2_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return K2_OK;
}

size_t k2_block_forward_static_ws_max_bytes(void) { return kStaticScratchBytes; }

int k2_block_forward_static_ws(const k2_block_cfg* cfg, const k2_block_weights* w, int B, int T, int N,
                               const float* hidden_in, float* hidden_out, const float* temb,
                               const float* position_ids, int pos_rows, int pos_cols, const uint8_t* mask,
                               void* stream) {
  int rc = validate_block_call(cfg, w, B, T, N, hidden_in, hidden_out, temb, position_ids, pos_rows, pos_cols);
  if (rc != K2_OK) return rc;
  const size_t need = k2_block_workspace_bytes(cfg, B, T, N);
  if (need > kStaticScratchBytes)
    return fail(K2_ERR_WORKSPACE, "this call needs %zu bytes of scratch; the static scratch holds %zu bytes", need,
                kStaticScratchBytes);
  void* ws = nullptr;
  if ((rc = static_scratch(&ws)) != K2_OK) return rc;
  g_err.clear();
  return block_run(cfg, w, B, T, N, hidden_in, hidden_out, temb, position_ids, mask, ws, nullptr, nullptr,
                   (hipStream_t)stream);
}

size_t k2_block_backward_workspace_bytes(const k2_block_cfg* cfg, int B, int T, int N) {
  if (!cfg || B < 0 || T < 0 || N < 0) return 0;
  return bwd_layout(cfg, B, T, N).total;
}

int k2_block_backward(const k2_block_cfg* cfg, const k2_block_weights* w, int B, int T, int N,
                      const float* hidden_in, const float* temb, const float* position_ids, int pos_rows,
                      int pos_cols, const uint8_t* mask, const float* grad_out, float* grad_in, float* grad_temb,
                      const k2_block_grads* grads, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = validate_block_call(cfg, w, B, T, N, hidden_in, grad_in, temb, position_ids, pos_rows, pos_cols);
  if (rc != K2_OK) return rc;
  if (!grad_out || !grad_in) return fail(K2_ERR_NULL, "grad_out / grad_in is NULL");
  if (!grads) return fail(K2_ERR_NULL, "grads is NULL (pass a struct of NULLs for no weight gradients)");
  if (grad_in == hidden_in || grad_in == grad_out) return fail(K2_ERR_CONFIG, "grad_in may not alias hidden_in or grad_out");
  if (cfg->hidden % 4 || cfg->hidden > 8192) return fail(K2_ERR_CONFIG, "the backward needs hidden <= 8192");
  {  // the attention backward addresses a batch row's query-side rows through one 32-bit-offset resource
    const long long L = (long long)T + N, nq = (long long)cfg->num_heads * cfg->head_dim;
    if (L * nq * (long long)dt_size(cfg->dtype) > 0x7FFFFFF0LL)
      return fail(K2_ERR_SHAPE, "sequence of %lld tokens too long for the backward: its query rows (%lld bytes per batch row) "
                  "exceed 2^31 - 16 bytes", L, L * nq * (long long)dt_size(cfg->dtype));
  }
  if (grad_temb && !w->scale_shift_table) return fail(K2_ERR_CONFIG, "grad_temb given for an unmodulated block");
  if (grads->scale_shift_table && !w->scale_shift_table)
    return fail(K2_ERR_CONFIG, "a scale_shift_table gradient asked of an unmodulated block");
  if ((rc = check_align("grad_out / grad_in / grad_temb / weight gradients",
                        {grad_out, grad_in, grad_temb, grads->scale_shift_table, grads->norm1_w, grads->norm2_w,
                         grads->norm_q_w, grads->norm_k_w, grads->to_q, grads->to_k, grads->to_v, grads->to_gate,
                         grads->to_out, grads->ff_gate, grads->ff_up, grads->ff_down})) != K2_OK)
    return rc;
  if ((rc = check_ws(workspace, workspace_bytes, bwd_layout(cfg, B, T, N).total)) != K2_OK) return rc;
  g_err.clear();
  return block_backward_run(cfg, w, B, T, N, hidden_in, temb, position_ids, mask, grad_out, grad_in, grad_temb, grads,
                            workspace, (hipStream_t)stream);
}

size_t k2_timestep_modulation_workspace_bytes(const k2_time_cfg* cfg, int B) {
  if (!cfg || B < 0) return 0;
  return time_layout(cfg, B).total;
}

int k2_timestep_modulation_forward(const k2_time_cfg* cfg, const k2_time_weights* w, int B, const float* timestep,
                                   float* temb, float* emb_out, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_time(cfg, w, B);
  if (rc != K2_OK) return rc;
  if (!timestep || !temb) return fail(K2_ERR_NULL, "timestep / temb is NULL");
  if ((rc = check_align("temb / emb_out", {temb, emb_out})) != K2_OK) return rc;
  if ((rc = check_ws(workspace, workspace_bytes, time_layout(cfg, B).total)) != K2_OK) return rc;
  g_err.clear();
  return time_run(cfg, w, B, timestep, temb, emb_out, workspace, (hipStream_t)stream);
}

size_t k2_text_fusion_workspace_bytes(const k2_text_cfg* cfg, int B, int T) {
  if (!cfg || B < 0 || T < 0) return 0;
  return text_layout(cfg, B, T).total;
}

int k2_text_fusion_forward(const k2_text_cfg* cfg, const k2_text_weights* w, int B, int T, const void* enc,
                           const uint8_t* mask, float* out, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_text(cfg, w, B, T);
  if (rc != K2_OK) return rc;
  if (!enc || !out) return fail(K2_ERR_NULL, "encoder_hidden_states / out is NULL");
  if ((rc = check_align("encoder_hidden_states / out", {enc, out})) != K2_OK) return rc;
  if ((rc = check_ws(workspace, workspace_bytes, text_layout(cfg, B, T).total)) != K2_OK) return rc;
  g_err.clear();
  return text_run(cfg, w, B, T, enc, mask, out, workspace, (hipStream_t)stream);
}

size_t k2_backbone_workspace_bytes(const k2_model_cfg* cfg, int B, int T, int N) {
  if (!cfg || B < 0 || T < 0 || N < 0) return 0;
  return model_layout(cfg, B, T, N).total;
}

size_t k2_backbone_cached_workspace_bytes(const k2_model_cfg* cfg, int B, int T, int N) {
  if (!cfg || B < 0 || T < 0 || N < 0) return 0;
  return model_layout(cfg, B, T, N, false).total;
}

size_t k2_text_embed_workspace_bytes(const k2_model_cfg* cfg, int B, int T) {
  if (!cfg || B < 0 || T < 0) return 0;
  return text_embed_layout(cfg, B, T).total;
}

int k2_text_embed(const k2_model_cfg* cfg, const k2_model_weights* w, int B, int T, const void* enc,
                  const uint8_t* mask, float* txt_h, void* workspace, size_t workspace_bytes, void* stream) {
  if (!cfg) return fail(K2_ERR_NULL, "model config is NULL");
  if (!w) return fail(K2_ERR_NULL, "model weights are NULL");
  int rc;
  if (cfg->text.block.dtype != cfg->block.dtype) return fail(K2_ERR_DTYPE, "text and block dtypes differ");
  if (cfg->block.hidden <= 0 || cfg->block.hidden % 8 || cfg->text.block.hidden % 8)
    return fail(K2_ERR_CONFIG, "hidden sizes must be positive multiples of 8");
  if ((rc = check_text(&cfg->text, &w->text, B, T)) != K2_OK) return rc;
  if (!w->txt_in_w) return fail(K2_ERR_NULL, "txt_in weight is NULL");
  if (!enc || !txt_h) return fail(K2_ERR_NULL, "encoder_hidden_states / txt_h is NULL");
  if ((rc = check_align("encoder_hidden_states / txt_h / txt_in", {enc, txt_h, w->txt_in_w, w->txt_in_b})) != K2_OK)
    return rc;
  if ((rc = check_ws(workspace, workspace_bytes, text_embed_layout(cfg, B, T).total)) != K2_OK) return rc;
  g_err.clear();
  return text_embed_run(cfg, w, B, T, enc, mask, txt_h, T, workspace, (hipStream_t)stream);
}

int backbone_run(const k2_model_cfg* cfg, const k2_model_weights* w, int B, int T, int N, const void* hidden_states,
                 const void* enc, const float* txt_cached, const float* timestep, const float* pos,
                 const uint8_t* mask, float* out, void* workspace, hipStream_t s);

// Validation shared by the backbone entry points; text: the call runs the text path on enc,
// otherwise txt_h holds its output.
int check_backbone_call(const k2_model_cfg* cfg, const k2_model_weights* w, int B, int T, int N,
                        const void* hidden_states, const void* enc, const float* txt_h, const float* timestep,
                        const float* pos, int pos_rows, int pos_cols, const float* out, bool text) {
  int rc = check_model(cfg, w, B, T, N, text);
  if (rc != K2_OK) return rc;
  if (!hidden_states || !timestep || !pos || !out)
    return fail(K2_ERR_NULL, "hidden_states / timestep / position_ids / out is NULL");
  if (T > 0 && text && !enc) return fail(K2_ERR_NULL, "encoder_hidden_states is NULL");
  if (T > 0 && !text && !txt_h) return fail(K2_ERR_NULL, "txt_h is NULL");
  if ((rc = check_align("hidden_states / encoder_hidden_states / txt_h / out", {hidden_states, enc, txt_h, out})) !=
      K2_OK)
    return rc;
  if (pos_rows != T + N || pos_cols != 3)
    return fail(K2_ERR_SHAPE, "position_ids must be (T + N, 3) = (%d, 3), got (%d, %d)", T + N, pos_rows, pos_cols);
  return K2_OK;
}

int k2_backbone_forward(const k2_model_cfg* cfg, const k2_model_weights* w, int B, int T, int N,
                        const void* hidden_states, const void* enc, const float* timestep, const float* pos,
                        int pos_rows, int pos_cols, const uint8_t* mask, float* out, void* workspace,
                        size_t workspace_bytes, void* stream) {
  int rc = check_backbone_call(cfg, w, B, T, N, hidden_states, enc, nullptr, timestep, pos, pos_rows, pos_cols, out,
                               true);
  if (rc != K2_OK) return rc;
  if ((rc = check_ws(workspace, workspace_bytes, model_layout(cfg, B, T, N).total)) != K2_OK) return rc;
  g_err.clear();
  return backbone_run(cfg, w, B, T, N, hidden_states, enc, nullptr, timestep, pos, mask, out, workspace,
                      (hipStream_t)stream);
}

int k2_backbone_forward_cached(const k2_model_cfg* cfg, const k2_model_weights* w, int B, int T, int N,
                               const void* hidden_states, const float* txt_h, const float* timestep,
                               const float* pos, int pos_rows, int pos_cols, const uint8_t* mask, float* out,
                               void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_backbone_call(cfg, w, B, T, N, hidden_states, nullptr, txt_h, timestep, pos, pos_rows, pos_cols,
                               out, false);
  if (rc != K2_OK) return rc;
  if ((rc = check_ws(workspace, workspace_bytes, model_layout(cfg, B, T, N, false).total)) != K2_OK) return rc;
  g_err.clear();
  return backbone_run(cfg, w, B, T, N, hidden_states, nullptr, txt_h, timestep, pos, mask, out, workspace,
                      (hipStream_t)stream);
}

// The backbone after validation (also the transformer call of the sampler steps). The text rows of
// h come from the text path on enc, or from txt_cached (B, T, hidden) when that is not NULL.
int backbone_run(const k2_model_cfg* cfg, const k2_model_weights* w, int B, int T, int N, const void* hidden_states,
                 const void* enc, const float* txt_cached, const float* timestep, const float* pos,
                 const uint8_t* mask, float* out, void* workspace, hipStream_t s) {
  int rc;
  const ModelLayout l = model_layout(cfg, B, T, N, txt_cached == nullptr);
  const int dt = cfg->block.dtype, H = cfg->block.hidden, hd = cfg->block.head_dim, L = T + N;
  const int C = cfg->in_channels;
  float* temb = (float*)at(workspace, l.temb);
  float* e = (float*)at(workspace, l.e);
  float* h = (float*)at(workspace, l.h);
  float* rc_ = (float*)at(workspace, l.rope);
  float* rs_ = rc_ + (size_t)L * (hd / 2);

  // time path: temb (B, 6H) shared by all blocks, e (B, H) for the final layer
  k2_time_cfg tc = {H, cfg->timestep_embed_dim, dt};
  if ((rc = time_run(&tc, &w->time, B, timestep, temb, e, at(workspace, l.time), s)) != K2_OK) return rc;

  // text path: text fusion -> txt_in into rows [0, T) of every batch row (its workspace regions
  // txt, txt_t, text are laid out as text_embed_layout's)
  if (T > 0) {
    if (txt_cached) {
      const size_t row = (size_t)T * H * sizeof(float);
      K2_RUN("copy", s, hipMemcpy2DAsync(h, (size_t)L * H * sizeof(float), txt_cached, row, row, B,
                                         hipMemcpyDeviceToDevice, s));
    } else if ((rc = text_embed_run(cfg, w, B, T, enc, mask, h, L, at(workspace, l.txt), s)) != K2_OK) {
      return rc;
    }
  }
  // image path: img_in into rows [T, L)
  {
    PlainArgs p = {};
    p.w = w->img_in_w; p.N = H; p.bias = w->img_in_b; p.outf = h; p.ldf = H;
    p.rows_per_b = N; p.out_rows_per_b = L; p.out_row_off = T;
    K2_RUN("gemm_plain", s, gemm_plain(dt, GemmA{hidden_states, C, B * N, C}, p, s));
  }
  // rotary table once for all blocks
  K2_RUN("rope", s, rope_table(pos, L, cfg->block.axes_dims[0], cfg->block.axes_dims[1], cfg->block.axes_dims[2],
                               cfg->block.rope_theta, rc_, rs_, s));
  void* bws = at(workspace, l.block);
  for (int i = 0; i < cfg->num_layers; ++i) {
    rc = block_run(&cfg->block, &w->blocks[i], B, T, N, h, h, temb, pos, mask, bws, rc_, rs_, s);
    if (rc != K2_OK) return rc;
  }
  // final layer over the image rows only
  float* fmod = (float*)at(workspace, l.fmod);
  void* xf = at(workspace, l.xf);
  K2_RUN("modulation", s, modulation(e, H, 0, w->final_table, fmod, B, 2, H, s));
  ModnormArgs mn = {};
  mn.in = h; mn.out = xf; mn.rows = B * N; mn.H = H;
  mn.rows_per_b = N; mn.in_rows_per_b = L; mn.in_row_off = T;
  mn.w = w->final_norm_w; mn.scale = fmod; mn.shift = fmod + H; mn.mod_stride = 2 * H; mn.eps = cfg->block.eps;
  K2_RUN("modnorm", s, modnorm(dt, mn, s));
  PlainArgs p = {};
  p.w = w->final_w; p.N = C; p.bias = w->final_b; p.outf = out; p.ldf = C;
  p.rows_per_b = B * N; p.out_rows_per_b = B * N; p.out_row_off = 0;
  K2_RUN("gemm_plain", s, gemm_plain(dt, GemmA{xf, H, B * N, H}, p, s));
  return K2_OK;
}

// ---------------------------------------------------------------------------------------------
// Sampler: flow-match Euler with the resolution-aware exponential time shift and guidance
// ([PIPELINE] Krea2Pipeline scheduler / is_distilled parameters, __call__ sigmas / guidance_scale)
// ---------------------------------------------------------------------------------------------
void k2_shift_cfg_default(k2_shift_cfg* c) {
  if (!c) return;
  c->base_shift = 0.5f;
  c->max_shift = 1.15f;
  c->base_image_seq_len = 256;
  c->max_image_seq_len = 6400;
  c->distilled_mu = 1.15f;
}

int k2_flow_sigmas(const k2_shift_cfg* cfg, int num_steps, int image_seq_len, int distilled, float* sigmas_out) {
  k2_shift_cfg d;
  k2_shift_cfg_default(&d);
  const k2_shift_cfg* c = cfg ? cfg : &d;
  if (!sigmas_out) return fail(K2_ERR_NULL, "sigmas_out is NULL");
  if (num_steps <= 0) return fail(K2_ERR_SHAPE, "num_steps must be >= 1");
  if (image_seq_len <= 0) return fail(K2_ERR_SHAPE, "image_seq_len must be >= 1");
  if (c->max_image_seq_len == c->base_image_seq_len)
    return fail(K2_ERR_CONFIG, "base_image_seq_len and max_image_seq_len must differ");
  double mu;
  if (distilled) {
    mu = c->distilled_mu;
  } else {
    const double slope = ((double)c->max_shift - c->base_shift) / ((double)c->max_image_seq_len - c->base_image_seq_len);
    mu = c->base_shift + slope * ((double)image_seq_len - c->base_image_seq_len);
  }
  const double em = std::exp(mu);
  for (int i = 0; i < num_steps; ++i) {
    // linspace(1, 1/N, N)
    const double sig = num_steps == 1 ? 1.0 : 1.0 + (1.0 / num_steps - 1.0) * i / (num_steps - 1);
    sigmas_out[i] = (float)(em / (em + (1.0 / sig - 1.0)));
  }
  sigmas_out[num_steps] = 0.0f;
  g_err.clear();
  return K2_OK;
}

int k2_cfg_euler_update(const float* x, float* x_out, const float* v_cond, const float* v_uncond, size_t n,
                        float guidance, float sigma, float sigma_next, void* stream) {
  if (n == 0) return K2_OK;
  if (!x || !x_out || !v_cond || (guidance > 0.0f && !v_uncond))
    return fail(K2_ERR_NULL, "x / x_out / v_cond (/ v_uncond when guidance > 0) is NULL");
  int rc;
  if ((rc = check_align("x / x_out / v_cond / v_uncond", {x, x_out, v_cond, v_uncond})) != K2_OK) return rc;
  if (!std::isfinite(guidance) || !std::isfinite(sigma) || !std::isfinite(sigma_next))
    return fail(K2_ERR_SHAPE, "guidance and sigmas must be finite");
  g_err.clear();
  hipStream_t s = (hipStream_t)stream;
  K2_RUN("cfg_euler", s, cfg_euler(x, x_out, v_cond, guidance > 0.0f ? v_uncond : nullptr, n, guidance,
                                   sigma_next - sigma, s));
  return K2_OK;
}

struct DenoiseLayout {
  size_t xin, v, t, model, total;
};
DenoiseLayout denoise_layout(const k2_model_cfg* c, int T, int N, int guided, bool text = true) {
  DenoiseLayout l = {};
  const int B = guided ? 2 : 1;
  const size_t nc = (size_t)N * c->in_channels;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  l.xin = take(B * nc * dt_size(c->block.dtype));
  l.v = take(B * nc * sizeof(float));
  l.t = take(B * sizeof(float));
  l.model = take(model_layout(c, B, T, N, text).total);
  l.total = off;
  return l;
}

size_t k2_denoise_workspace_bytes(const k2_model_cfg* cfg, int T, int N, int guided) {
  if (!cfg || T < 0 || N < 0) return 0;
  return denoise_layout(cfg, T, N, guided != 0).total;
}

size_t k2_denoise_cached_workspace_bytes(const k2_model_cfg* cfg, int T, int N, int guided) {
  if (!cfg || T < 0 || N < 0) return 0;
  return denoise_layout(cfg, T, N, guided != 0, false).total;
}

// One sampler step: the transformer on enc (text path run here) or on the cached text rows txt_h.
int denoise_call(const k2_model_cfg* cfg, const k2_model_weights* w, int T, int N, float* latents, const void* enc,
                 const float* txt_h, bool text, const uint8_t* mask, const float* pos, int pos_rows, int pos_cols,
                 float sigma, float sigma_next, float guidance, void* workspace, size_t workspace_bytes,
                 void* stream) {
  const int guided = guidance > 0.0f, B = guided ? 2 : 1;
  int rc = check_model(cfg, w, B, T, N, text);
  if (rc != K2_OK) return rc;
  if (!latents || !pos) return fail(K2_ERR_NULL, "latents / position_ids is NULL");
  if (T > 0 && text && !enc) return fail(K2_ERR_NULL, "encoder_hidden_states is NULL");
  if (T > 0 && !text && !txt_h) return fail(K2_ERR_NULL, "txt_h is NULL");
  if ((rc = check_align("latents / encoder_hidden_states / txt_h", {latents, enc, txt_h})) != K2_OK) return rc;
  if (pos_rows != T + N || pos_cols != 3)
    return fail(K2_ERR_SHAPE, "position_ids must be (T + N, 3) = (%d, 3), got (%d, %d)", T + N, pos_rows, pos_cols);
  if (!std::isfinite(guidance) || !std::isfinite(sigma) || !std::isfinite(sigma_next))
    return fail(K2_ERR_SHAPE, "guidance and sigmas must be finite");
  const DenoiseLayout l = denoise_layout(cfg, T, N, guided, text);
  if ((rc = check_ws(workspace, workspace_bytes, l.total)) != K2_OK) return rc;
  g_err.clear();

  hipStream_t s = (hipStream_t)stream;
  const int dt = cfg->block.dtype;
  const size_t nc = (size_t)N * cfg->in_channels, es = dt_size(dt);
  char* xin = at(workspace, l.xin);
  float* v = (float*)at(workspace, l.v);
  float* t = (float*)at(workspace, l.t);
  // the transformer input: the latents in the operand dtype, once per guidance branch
  for (int b = 0; b < B; ++b) K2_RUN("convert", s, from_f32(dt, latents, xin + b * nc * es, nc, s));
  K2_RUN("fill", s, fill_f32(t, B, sigma, s));
  if ((rc = backbone_run(cfg, w, B, T, N, xin, text ? enc : nullptr, text ? nullptr : txt_h, t, pos, mask, v,
                         at(workspace, l.model), s)) != K2_OK)
    return rc;
  K2_RUN("cfg_euler", s, cfg_euler(latents, latents, v, guided ? v + nc : nullptr, nc, guidance, sigma_next - sigma, s));
  return K2_OK;
}

int k2_denoise_step(const k2_model_cfg* cfg, const k2_model_weights* w, int T, int N, float* latents, const void* enc,
                    const uint8_t* mask, const float* pos, int pos_rows, int pos_cols, float sigma, float sigma_next,
                    float guidance, void* workspace, size_t workspace_bytes, void* stream) {
  return denoise_call(cfg, w, T, N, latents, enc, nullptr, true, mask, pos, pos_rows, pos_cols, sigma, sigma_next,
                      guidance, workspace, workspace_bytes, stream);
}

int k2_denoise_step_cached(const k2_model_cfg* cfg, const k2_model_weights* w, int T, int N, float* latents,
                           const float* txt_h, const uint8_t* mask, const float* pos, int pos_rows, int pos_cols,
                           float sigma, float sigma_next, float guidance, void* workspace, size_t workspace_bytes,
                           void* stream) {
  return denoise_call(cfg, w, T, N, latents, nullptr, txt_h, false, mask, pos, pos_rows, pos_cols, sigma, sigma_next,
                      guidance, workspace, workspace_bytes, stream);
}

const char* k2_last_error(void) { return g_err.c_str(); }

int k2_mfma_rate_probe(int iters, int blocks, float* out, void* stream) {
  if (!out) return fail(K2_ERR_NULL, "out is NULL");
  if (iters <= 0 || blocks <= 0 || blocks > 65535) return fail(K2_ERR_SHAPE, "need iters >= 1 and 1 <= blocks <= 65535");
  int rc;
  if ((rc = check_align("out", {out})) != K2_OK) return rc;
  g_err.clear();
  K2_RUN("mfma_probe", (hipStream_t)stream, mfma_probe(iters, blocks, out, (hipStream_t)stream));
  return K2_OK;
}

void k2_profile_enable(int enable) {
  std::lock_guard<std::mutex> lk(g_pm);
  g_prof.store(enable != 0);
}

void k2_profile_filter(const char* kernel) {
  std::lock_guard<std::mutex> lk(g_pm);
  g_pfilter = kernel ? kernel : "";
}

void k2_profile_reset(void) {
  std::lock_guard<std::mutex> lk(g_pm);
  for (auto& ev : g_pev) {
    g_pool.push_back(ev.a);
    g_pool.push_back(ev.b);
  }
  g_pev.clear();
}

int k2_profile_query(const char* kernel, double* total_ms, int* launches) {
  if (!kernel || !total_ms || !launches) return fail(K2_ERR_NULL, "NULL argument");
  std::lock_guard<std::mutex> lk(g_pm);
  double tot = 0.0;
  int n = 0;
  for (auto& ev : g_pev) {
    if (ev.name != kernel) continue;
    if (hipEventSynchronize(ev.b) != hipSuccess) return fail(K2_ERR_HIP, "event synchronize failed");
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, ev.a, ev.b) != hipSuccess) return fail(K2_ERR_HIP, "event elapsed time failed");
    tot += ms;
    ++n;
  }
  *total_ms = tot;
  *launches = n;
  return K2_OK;
}

}  // extern "C"
