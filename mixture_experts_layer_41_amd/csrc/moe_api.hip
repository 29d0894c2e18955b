// C ABI of the MoE layer library: argument validation, exact capacity,
// workspace planning and the launch sequences of the entry points.
// Nothing here allocates device memory or synchronises; every launch goes to
// the caller's stream.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>

#include "moe_internal.h"

using namespace moe;

namespace {

constexpr size_t kAlign = 256;

// Carves aligned regions out of a workspace; with base == nullptr it only
// measures.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <class T>
  T* take(size_t n) {
    off = (off + kAlign - 1) / kAlign * kAlign;
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += n * sizeof(T);
    return p;
  }
};

size_t act_bytes(const moe_config& c) { return c.dtype == MOE_DTYPE_BF16 ? 2 : 4; }
int64_t route_blocks(const moe_config& c) {
  const int BT = route_block_tokens(c.n_tokens, c.n_experts);
  return (c.n_tokens + BT - 1) / BT;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// The router's score modifiers; temperature 0 means 1.
RouterMod router_mod(const moe_config& c, const float* bias, const float* noise) {
  RouterMod m;
  m.bias = bias;
  m.noise = noise;
  m.inv_tau = c.router_temperature == 0.f ? 1.f : 1.f / c.router_temperature;
  m.scores_out = nullptr;
  return m;
}

moe_status check_config(const moe_config* c) {
  if (c == nullptr) return MOE_ERR_INVALID_ARG;
  if (c->n_tokens < 1 || c->d_model < 8 || c->d_ffn < 8 || c->n_experts < 1 || c->top_k < 1 ||
      c->top_k > c->n_experts || c->n_shared < 0)
    return MOE_ERR_INVALID_ARG;
  if (c->weight_format != MOE_WEIGHTS_ACT && c->weight_format != MOE_WEIGHTS_INT8)
    return MOE_ERR_INVALID_ARG;
  if (c->dtype != MOE_DTYPE_F32 && c->dtype != MOE_DTYPE_BF16) return MOE_ERR_INVALID_ARG;
  if (c->act != MOE_ACT_GELU && c->act != MOE_ACT_SWIGLU) return MOE_ERR_INVALID_ARG;
  if (c->add_residual != 0 && c->add_residual != 1) return MOE_ERR_INVALID_ARG;
  if (std::isnan(c->capacity_factor) || std::isinf(c->capacity_factor) ||
      c->capacity_factor > 1073741824.0)
    return MOE_ERR_INVALID_ARG;
  if (c->router_temperature != 0.f &&
      !(c->router_temperature > 0.f && std::isfinite(c->router_temperature) &&
        std::isfinite(1.f / c->router_temperature)))
    return MOE_ERR_INVALID_ARG;
  if (c->d_model % 8 != 0 || c->d_ffn % 8 != 0) return MOE_ERR_UNSUPPORTED;
  if (c->n_experts > kMaxExperts || c->n_shared > 64) return MOE_ERR_UNSUPPORTED;
  // INT8 expert weights: bf16 activations; shapes the dequantizing tiled
  // GEMM covers for every activation (K tile 64, output tiles of 128)
  if (c->weight_format == MOE_WEIGHTS_INT8 &&
      (c->dtype != MOE_DTYPE_BF16 || c->d_model % 128 != 0 || c->d_ffn % 128 != 0))
    return MOE_ERR_UNSUPPORTED;
  // row indices are int32
  if (c->n_tokens * (int64_t)c->top_k >= (int64_t)1 << 31) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)c->d_ffn * (c->n_shared > 1 ? c->n_shared : 1) >= (int64_t)1 << 30)
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// C = ceil(cf * T * k / E) on the exact binary64 value of cf; -1 = no limit.
int64_t exact_capacity(const moe_config& c) {
  const double cf = c.capacity_factor;
  if (!(cf > 0.0)) return -1;
  int e2 = 0;
  const double m = std::frexp(cf, &e2);                      // cf = m * 2^e2, m in [0.5, 1)
  const unsigned __int128 M = (unsigned __int128)std::ldexp(m, 53);  // exact 53-bit integer
  const unsigned __int128 N = (unsigned __int128)(c.n_tokens * (int64_t)c.top_k);
  const int shift = e2 - 53;                                 // cf = M * 2^shift
  unsigned __int128 num = M * N;
  unsigned __int128 den = (unsigned __int128)c.n_experts;
  if (shift >= 0) {
    num <<= shift;  // cf <= 2^30 keeps this below 2^115
  } else {
    if (-shift >= 100) return 1;  // cf*T*k/E < 1 and > 0
    den <<= -shift;
  }
  return (int64_t)((num + den - 1) / den);
}

struct RouteWs {
  RouteStats st;
  size_t bytes;
};

RouteWs plan_route(const moe_config& c, void* ws) {
  Carver cv(ws);
  const int64_t nb = route_blocks(c);
  RouteWs r;
  r.st.cnt = cv.take<int32_t>(nb * c.n_experts);
  r.st.psum = cv.take<float>(nb * c.n_experts);
  r.st.zsum = cv.take<float>(nb);
  r.st.bad = cv.take<int32_t>(nb);
  r.st.logit_part = cv.take<float>(router_scratch_bytes(c) / sizeof(float));
  r.bytes = cv.off;
  return r;
}

moe_status ws_check(void* ws, size_t* ws_bytes, size_t need) {
  if (ws_bytes == nullptr) return MOE_ERR_INVALID_ARG;
  if (ws == nullptr) {
    *ws_bytes = need;
    return MOE_OK;
  }
  if (!aligned16(ws)) return MOE_ERR_INVALID_ARG;
  if (*ws_bytes < need) {
    *ws_bytes = need;
    return MOE_ERR_WORKSPACE;
  }
  return MOE_OK;
}

#define MOE_HIP_TRY(expr)                          \
  do {                                             \
    if ((expr) != hipSuccess) return MOE_ERR_HIP;  \
  } while (0)

}  // namespace

extern "C" {

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

moe_status moe_route(const moe_config* cfg, const void* x, const void* w_router,
                     const float* router_bias, const float* router_noise, int32_t* topk_idx,
                     float* topk_w, float* token_lse, void* ws, size_t* ws_bytes,
                     hipStream_t stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  const RouteWs plan = plan_route(*cfg, nullptr);
  if (ws != nullptr) {
    if (!x || !w_router || !topk_idx || !topk_w) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(w_router) || !aligned4(router_noise)) return MOE_ERR_INVALID_ARG;
  }
  st = ws_check(ws, ws_bytes, plan.bytes);
  if (st != MOE_OK || ws == nullptr) return st;
  const RouteWs r = plan_route(*cfg, ws);
  MOE_HIP_TRY(launch_router(*cfg, x, w_router, router_mod(*cfg, router_bias, router_noise), topk_idx,
                            topk_w, token_lse, r.st, stream));
  return MOE_OK;
}

moe_status moe_permute(const moe_config* cfg, const int32_t* topk_idx, const float* topk_w,
                       const void* x, int32_t* expert_counts, int32_t* expert_offsets,
                       int32_t* perm_token, float* perm_w, int32_t* inv_row, void* x_perm,
                       int32_t* n_dropped, void* ws, size_t* ws_bytes, hipStream_t stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  const int64_t nb = route_blocks(*cfg);
  auto plan = [&](void* base, RouteStats& rs, void*& scratch) {
    Carver cv(base);
    rs.cnt = cv.take<int32_t>(nb * cfg->n_experts);
    rs.bad = cv.take<int32_t>(nb);
    rs.psum = nullptr;
    rs.zsum = nullptr;
    scratch = cv.take<char>(permute_scratch_bytes(*cfg));
    return cv.off;
  };
  RouteStats rs{};
  void* scratch = nullptr;
  const size_t need = plan(nullptr, rs, scratch);
  if (ws != nullptr) {
    if (!topk_idx || !expert_counts || !expert_offsets || !perm_token || !inv_row || !n_dropped)
      return MOE_ERR_INVALID_ARG;
    if (perm_w && !topk_w) return MOE_ERR_INVALID_ARG;
    if (x_perm && (!x || !aligned16(x) || !aligned16(x_perm))) return MOE_ERR_INVALID_ARG;
  }
  st = ws_check(ws, ws_bytes, need);
  if (st != MOE_OK || ws == nullptr) return st;
  plan(ws, rs, scratch);
  const int64_t cap = exact_capacity(*cfg);
  PermuteOut po{expert_counts, expert_offsets, n_dropped, perm_token, perm_w, inv_row};
  MOE_HIP_TRY(launch_histogram(*cfg, topk_idx, rs, stream));
  MOE_HIP_TRY(launch_permute(*cfg, rs, po, cap, topk_idx, topk_w, x, x_perm, nullptr, scratch,
                             stream));
  return MOE_OK;
}

}  // extern "C"

namespace {

// moe_expert_ffn and moe_expert_ffn_int8 (w1_scale / w2_scale non-null with
// INT8 codes in w1 / w2).
moe_status expert_ffn(const moe_config* cfg, int32_t n_groups, int32_t n_seg, int64_t rows_max,
                      const void* a, const int32_t* a_rows, const int32_t* group_offsets,
                      const void* w1, const float* w1_scale, const void* b1, const void* w2,
                      const float* w2_scale, const void* b2, void* out, void* ws,
                      size_t* ws_bytes, hipStream_t stream) {
  const bool q8 = cfg->weight_format == MOE_WEIGHTS_INT8;
  if (n_groups < 1 || n_seg < 1 || n_seg > 64 || rows_max < 0) return MOE_ERR_INVALID_ARG;
  if (group_offsets == nullptr && n_groups != 1) return MOE_ERR_INVALID_ARG;
  if (rows_max >= (int64_t)1 << 31) return MOE_ERR_UNSUPPORTED;
  const int64_t hw = (int64_t)n_seg * cfg->d_ffn;  // intermediate width
  Carver cv(nullptr);
  cv.take<char>((size_t)rows_max * hw * act_bytes(*cfg));
  const size_t need = cv.off;
  if (ws != nullptr) {
    if (!a || !w1 || !w2 || !out) return MOE_ERR_INVALID_ARG;
    if (!aligned16(a) || !aligned16(w1) || !aligned16(w2) || !aligned16(out))
      return MOE_ERR_INVALID_ARG;
    if (q8 && (!w1_scale || !w2_scale || !aligned4(w1_scale) || !aligned4(w2_scale)))
      return MOE_ERR_INVALID_ARG;
  }
  moe_status st = ws_check(ws, ws_bytes, need);
  if (st != MOE_OK || ws == nullptr) return st;
  if (rows_max == 0) return MOE_OK;
  Carver c2(ws);
  void* H = c2.take<char>((size_t)rows_max * hw * act_bytes(*cfg));

  GemmDesc up{};
  up.a = a;
  up.a_rows = a_rows;
  up.lda = cfg->d_model;
  up.group_off = group_offsets;
  up.n_groups = n_groups;
  up.n_seg = n_seg;
  up.rows_max = rows_max;
  up.w = w1;
  up.w_scale = q8 ? w1_scale : nullptr;
  up.bias = b1;
  up.d = cfg->d_model;
  up.f = cfg->d_ffn;
  up.act = cfg->act;
  up.out = H;
  up.ldo = hw;
  MOE_HIP_TRY(launch_gemm(*cfg, kGemmUp, up, stream));
  GemmDesc dn = up;
  dn.a = H;
  dn.a_rows = nullptr;
  dn.lda = hw;
  dn.w = w2;
  dn.w_scale = q8 ? w2_scale : nullptr;
  dn.bias = b2;
  dn.out = out;
  dn.ldo = cfg->d_model;
  MOE_HIP_TRY(launch_gemm(*cfg, kGemmDown, dn, stream));
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_expert_ffn(const moe_config* cfg, int32_t n_groups, int32_t n_seg,
                          int64_t rows_max, const void* a, const int32_t* a_rows,
                          const int32_t* group_offsets, const void* w1, const void* b1,
                          const void* w2, const void* b2, void* out, void* ws,
                          size_t* ws_bytes, hipStream_t stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (cfg->weight_format != MOE_WEIGHTS_ACT) return MOE_ERR_INVALID_ARG;
  return expert_ffn(cfg, n_groups, n_seg, rows_max, a, a_rows, group_offsets, w1, nullptr, b1, w2,
                    nullptr, b2, out, ws, ws_bytes, stream);
}

moe_status moe_expert_ffn_int8(const moe_config* cfg, int32_t n_groups, int32_t n_seg,
                               int64_t rows_max, const void* a, const int32_t* a_rows,
                               const int32_t* group_offsets, const int8_t* w1,
                               const float* w1_scale, const void* b1, const int8_t* w2,
                               const float* w2_scale, const void* b2, void* out, void* ws,
                               size_t* ws_bytes, hipStream_t stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (cfg->weight_format != MOE_WEIGHTS_INT8) return MOE_ERR_INVALID_ARG;
  return expert_ffn(cfg, n_groups, n_seg, rows_max, a, a_rows, group_offsets, w1, w1_scale, b1,
                    w2, w2_scale, b2, out, ws, ws_bytes, stream);
}

moe_status moe_combine(const moe_config* cfg, const void* y_perm, const int32_t* inv_row,
                       const float* topk_w, const void* shared_y, const void* residual,
                       void* y, hipStream_t stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!y_perm || !inv_row || !topk_w || !y) return MOE_ERR_INVALID_ARG;
  if (!aligned16(y) || !aligned16(y_perm) || (shared_y && !aligned16(shared_y)) ||
      (residual && !aligned16(residual)))
    return MOE_ERR_INVALID_ARG;
  MOE_HIP_TRY(launch_combine(*cfg, y_perm, inv_row, topk_w, shared_y, residual, y, stream));
  return MOE_OK;
}

moe_status moe_aux_stats(const moe_config* cfg, const int32_t* expert_counts,
                         const int32_t* n_dropped, const void* route_ws, size_t route_ws_bytes,
                         moe_aux* aux, hipStream_t stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!expert_counts || !n_dropped || !route_ws || !aux) return MOE_ERR_INVALID_ARG;
  const RouteWs plan = plan_route(*cfg, nullptr);
  if (route_ws_bytes < plan.bytes) return MOE_ERR_WORKSPACE;
  const RouteWs r = plan_route(*cfg, const_cast<void*>(route_ws));
  MOE_HIP_TRY(launch_aux(*cfg, r.st, expert_counts, n_dropped, exact_capacity(*cfg), aux, stream));
  return MOE_OK;
}

// The forward of moe_forward and moe_forward_train (saved != null: the
// routing results, scores, lse, permutation and expert outputs go to the
// caller's buffers).
static moe_status forward_impl(const moe_config* cfg, const moe_weights* w, const void* x,
                               const float* router_noise, void* y, int32_t* topk_idx,
                               float* topk_w, int32_t* expert_counts, moe_aux* aux,
                               const moe_saved* saved, void* ws, size_t* ws_bytes,
                               hipStream_t stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  const moe_config& c = *cfg;
  const int64_t T = c.n_tokens, R = T * c.top_k, nb = route_blocks(c);
  const int E = c.n_experts, S = c.n_shared, d = c.d_model, f = c.d_ffn;
  const size_t ab = act_bytes(c);

  struct Plan {
    RouteStats rs;
    PermuteOut po;
    void* scratch;
    int32_t* idx;
    float* wts;
    void *H, *y_perm, *Hs, *shared_y;
  };
  auto plan = [&](void* base, Plan& p) {
    Carver cv(base);
    p.rs.cnt = cv.take<int32_t>(nb * E);
    p.rs.psum = cv.take<float>(nb * E);
    p.rs.zsum = cv.take<float>(nb);
    p.rs.bad = nullptr;
    p.rs.logit_part = cv.take<float>(router_scratch_bytes(c) / sizeof(float));
    p.scratch = cv.take<char>(permute_scratch_bytes(c));
    p.po.counts = cv.take<int32_t>(E);
    p.po.offsets = cv.take<int32_t>(E + 1);
    p.po.n_dropped = cv.take<int32_t>(1);
    p.po.perm_w = nullptr;
    p.idx = cv.take<int32_t>(R);
    p.wts = cv.take<float>(R);
    p.po.perm_token = cv.take<int32_t>(R);
    p.po.inv_row = cv.take<int32_t>(R);
    p.H = cv.take<char>((size_t)R * f * ab);
    p.y_perm = cv.take<char>((size_t)R * d * ab);
    p.Hs = S ? cv.take<char>((size_t)T * S * f * ab) : nullptr;
    p.shared_y = S ? cv.take<char>((size_t)T * d * ab) : nullptr;
    return cv.off;
  };
  Plan p{};
  const size_t need = plan(nullptr, p);
  if (ws != nullptr) {
    if (!w || !x || !y || !w->w_router || !w->w1 || !w->w2) return MOE_ERR_INVALID_ARG;
    if (S > 0 && (!w->shared_w1 || !w->shared_w2)) return MOE_ERR_INVALID_ARG;
    if (!aligned4(router_noise)) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(y) || !aligned16(w->w_router) || !aligned16(w->w1) ||
        !aligned16(w->w2) || (S > 0 && (!aligned16(w->shared_w1) || !aligned16(w->shared_w2))))
      return MOE_ERR_INVALID_ARG;
    if (c.weight_format == MOE_WEIGHTS_INT8) {
      if (!w->w1_scale || !w->w2_scale || !aligned4(w->w1_scale) || !aligned4(w->w2_scale))
        return MOE_ERR_INVALID_ARG;
      if (S > 0 && (!w->shared_w1_scale || !w->shared_w2_scale || !aligned4(w->shared_w1_scale) ||
                    !aligned4(w->shared_w2_scale)))
        return MOE_ERR_INVALID_ARG;
    }
  }
  st = ws_check(ws, ws_bytes, need);
  if (st != MOE_OK || ws == nullptr) return st;
  plan(ws, p);
  if (topk_idx) p.idx = topk_idx;
  if (topk_w) p.wts = topk_w;
  if (expert_counts) p.po.counts = expert_counts;
  RouterMod rm = router_mod(c, w->router_bias, router_noise);
  float* lse_out = nullptr;
  if (saved) {
    p.idx = saved->topk_idx;
    p.wts = saved->topk_w;
    p.po.counts = saved->expert_counts;
    p.po.offsets = saved->expert_offsets;
    p.po.perm_token = saved->perm_token;
    p.po.inv_row = saved->inv_row;
    p.y_perm = saved->y_perm;
    rm.scores_out = saved->scores;
    lse_out = saved->token_lse;
  }
  const int64_t cap = exact_capacity(c);
  const bool q8 = c.weight_format == MOE_WEIGHTS_INT8;

  MOE_HIP_TRY(launch_router(c, x, w->w_router, rm, p.idx, p.wts, lse_out, p.rs, stream));
  MOE_HIP_TRY(launch_permute(c, p.rs, p.po, cap, p.idx, nullptr, nullptr, nullptr, aux, p.scratch,
                             stream));

  GemmDesc up{};
  up.a = x;
  up.a_rows = p.po.perm_token;
  up.lda = d;
  up.group_off = p.po.offsets;
  up.n_groups = E;
  up.n_seg = 1;
  up.rows_max = R;
  up.w = w->w1;
  up.w_scale = q8 ? w->w1_scale : nullptr;
  up.bias = w->b1;
  up.d = d;
  up.f = f;
  up.act = c.act;
  up.out = p.H;
  up.ldo = f;
  if (saved) {
    up.preact = saved->preact;
    up.ldp = c.act == MOE_ACT_SWIGLU ? 2 * f : f;
  }
  MOE_HIP_TRY(launch_gemm(c, kGemmUp, up, stream));
  GemmDesc dn = up;
  dn.a = p.H;
  dn.a_rows = nullptr;
  dn.lda = f;
  dn.w = w->w2;
  dn.w_scale = q8 ? w->w2_scale : nullptr;
  dn.bias = w->b2;
  dn.out = p.y_perm;
  dn.ldo = d;
  dn.preact = nullptr;
  MOE_HIP_TRY(launch_gemm(c, kGemmDown, dn, stream));

  if (S > 0) {
    GemmDesc su{};
    su.a = x;
    su.a_rows = nullptr;
    su.lda = d;
    su.group_off = nullptr;  // one dense group of T rows
    su.n_groups = 1;
    su.n_seg = S;
    su.rows_max = T;
    su.w = w->shared_w1;
    su.w_scale = q8 ? w->shared_w1_scale : nullptr;
    su.bias = w->shared_b1;
    su.d = d;
    su.f = f;
    su.act = c.act;
    su.out = p.Hs;
    su.ldo = (int64_t)S * f;
    if (saved) {
      su.preact = saved->shared_preact;
      su.ldp = (int64_t)S * (c.act == MOE_ACT_SWIGLU ? 2 * f : f);
    }
    MOE_HIP_TRY(launch_gemm(c, kGemmUp, su, stream));
    GemmDesc sd = su;
    sd.a = p.Hs;
    sd.lda = (int64_t)S * f;
    sd.w = w->shared_w2;
    sd.w_scale = q8 ? w->shared_w2_scale : nullptr;
    sd.bias = w->shared_b2;
    sd.out = p.shared_y;
    sd.ldo = d;
    sd.preact = nullptr;
    MOE_HIP_TRY(launch_gemm(c, kGemmDown, sd, stream));
  }
  MOE_HIP_TRY(launch_combine(c, p.y_perm, p.po.inv_row, p.wts, p.shared_y,
                             c.add_residual ? x : nullptr, y, stream));
  return MOE_OK;
}

moe_status moe_forward(const moe_config* cfg, const moe_weights* w, const void* x,
                       const float* router_noise, void* y, int32_t* topk_idx, float* topk_w,
                       int32_t* expert_counts, moe_aux* aux, void* ws, size_t* ws_bytes,
                       hipStream_t stream) {
  return forward_impl(cfg, w, x, router_noise, y, topk_idx, topk_w, expert_counts, aux, nullptr, ws,
                      ws_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// moe_forward_static: the scratch memory of moe_forward in a static device
// array.  Each GPU the library runs on holds its own copy (the code object's
// variable) from the first call on that device until the process ends.  In
// host code the array's name is only a host-side stand-in: its device
// address is looked up once per device with hipGetSymbolAddress (with that
// device current) and only that address is ever handed to kernels.

static __device__ __align__(256) unsigned char scratch[MOE_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device

moe_status static_scratch(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_forward_static(const moe_config* cfg, const moe_weights* w, const void* x,
                              const float* router_noise, void* y, int32_t* topk_idx, float* topk_w,
                              int32_t* expert_counts, moe_aux* aux, hipStream_t stream) {
  void* ws = nullptr;
  const moe_status st = static_scratch(&ws);
  if (st != MOE_OK) return st;
  // the workspace check of the forward rejects a layer whose scratch need
  // exceeds the array (MOE_ERR_WORKSPACE) before anything is launched; no
  // kernel of the forward needs its scratch memory cleared
  size_t n = MOE_STATIC_SCRATCH_BYTES;
  return forward_impl(cfg, w, x, router_noise, y, topk_idx, topk_w, expert_counts, aux, nullptr, ws,
                      &n, stream);
}

// Training needs bf16 activations and activation-dtype expert weights.
static moe_status check_train(const moe_config* cfg) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (cfg->dtype != MOE_DTYPE_BF16 || cfg->weight_format != MOE_WEIGHTS_ACT)
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

static bool saved_ok(const moe_saved* sv, int S) {
  return sv && sv->scores && sv->token_lse && sv->topk_idx && sv->topk_w && sv->expert_counts &&
         sv->expert_offsets && sv->perm_token && sv->inv_row && sv->y_perm && sv->preact &&
         aligned16(sv->preact) &&
         (S == 0 || (sv->shared_preact && aligned16(sv->shared_preact))) && aligned4(sv->scores) &&
         aligned4(sv->token_lse) && aligned4(sv->topk_idx) && aligned4(sv->topk_w) &&
         aligned4(sv->expert_counts) && aligned4(sv->expert_offsets) && aligned4(sv->perm_token) &&
         aligned4(sv->inv_row) && aligned16(sv->y_perm);
}

moe_status moe_forward_train(const moe_config* cfg, const moe_weights* w, const void* x,
                             const float* router_noise, void* y, const moe_saved* saved,
                             moe_aux* aux, void* ws, size_t* ws_bytes, hipStream_t stream) {
  moe_status st = check_train(cfg);
  if (st != MOE_OK) return st;
  if (ws != nullptr && !saved_ok(saved, cfg->n_shared)) return MOE_ERR_INVALID_ARG;
  return forward_impl(cfg, w, x, router_noise, y, nullptr, nullptr, nullptr, aux,
                      ws != nullptr ? saved : nullptr, ws, ws_bytes, stream);
}

moe_status moe_backward(const moe_config* cfg, const moe_weights* w, const void* x,
                        const moe_saved* sv, const void* dy, const moe_loss_weights* lw_in,
                        const moe_grads* g, void* ws, size_t* ws_bytes, hipStream_t stream) {
  moe_status st = check_train(cfg);
  if (st != MOE_OK) return st;
  moe_loss_weights lw{0.01, 0.001, 0.0, 0.0};  // the pages' training loss
  if (lw_in) lw = *lw_in;
  if (!std::isfinite(lw.load_balance) || !std::isfinite(lw.z_loss) ||
      !std::isfinite(lw.lb_squares) || !std::isfinite(lw.kl_uniform))
    return MOE_ERR_INVALID_ARG;
  const moe_config& c = *cfg;
  const int64_t T = c.n_tokens, R = T * c.top_k;
  const int E = c.n_experts, S = c.n_shared, d = c.d_model, f = c.d_ffn;
  const int w1r = c.act == MOE_ACT_SWIGLU ? 2 * f : f;
  constexpr int kPad = 64;  // K tile of the weight-gradient GEMM
  const int64_t Rp = (R + (int64_t)kPad * E + kPad - 1) / kPad * kPad;  // padded columns, bound
  const int64_t Tp = (T + kPad - 1) / kPad * kPad;
  const int nsplit = router_wgrad_splits(E, d, T);
  const bool p_terms = lw.lb_squares != 0.0 || lw.kl_uniform != 0.0;
  // split weight-gradient products share one partial buffer (same stream)
  size_t wg_part = 0;
  auto wg_need = [&](int M, int N, int batches, int64_t K, bool grouped) {
    const WgradPlan pl = wgrad_plan(M, N, batches, grouped ? K / batches : K);
    wg_part = std::max(wg_part, wgrad_partial_floats(pl, M, N, batches));
  };
  wg_need(d, f, E, Rp, true);
  wg_need(w1r, d, E, Rp, true);
  if (S > 0) {
    wg_need(d, f, S, Tp, false);
    wg_need(w1r, d, S, Tp, false);
  }

  struct Plan {
    void *dO, *W2t, *W1t, *dH, *dA, *dXr, *dOt, *Ht, *dAt, *Xt;
    float *dl, *wr_part, *aux_dp, *wg_part;
    int32_t *poff, *colrow;
    void *Ws2t, *Ws1t, *dHs, *dAs, *dXs, *dyt, *Hst, *dAst, *xt;
  };
  auto plan = [&](void* base, Plan& p) {
    Carver cv(base);
    p.dO = cv.take<uint16_t>(R * d);
    p.dl = cv.take<float>(T * E);
    p.aux_dp = cv.take<float>(E);  // the size does not depend on the loss weights
    p.wr_part = cv.take<float>((size_t)nsplit * router_wgrad_split_ld(E, d));
    p.W2t = cv.take<uint16_t>((size_t)E * f * d);
    p.W1t = cv.take<uint16_t>((size_t)E * d * w1r);
    p.dH = cv.take<uint16_t>(R * f);
    p.dA = cv.take<uint16_t>(R * w1r);
    p.dXr = cv.take<uint16_t>(R * d);
    p.poff = cv.take<int32_t>(E + 1);
    p.colrow = cv.take<int32_t>(Rp);
    p.dOt = cv.take<uint16_t>(d * Rp);
    p.Ht = cv.take<uint16_t>(f * Rp);
    p.dAt = cv.take<uint16_t>(w1r * Rp);
    p.Xt = cv.take<uint16_t>(d * Rp);
    p.wg_part = cv.take<float>(wg_part);
    if (S > 0) {
      p.Ws2t = cv.take<uint16_t>((size_t)S * f * d);
      p.Ws1t = cv.take<uint16_t>((size_t)S * d * w1r);
      p.dHs = cv.take<uint16_t>(T * S * f);
      p.dAs = cv.take<uint16_t>(T * S * w1r);
      p.dXs = cv.take<uint16_t>(T * d);
      p.dyt = cv.take<uint16_t>(d * Tp);
      p.Hst = cv.take<uint16_t>(S * f * Tp);
      p.dAst = cv.take<uint16_t>(S * w1r * Tp);
      p.xt = cv.take<uint16_t>(d * Tp);
    }
    return cv.off;
  };
  Plan p{};
  const size_t need = plan(nullptr, p);
  if (ws != nullptr) {
    if (!w || !x || !dy || !g || !saved_ok(sv, S) || !w->w_router || !w->w1 || !w->w2)
      return MOE_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(dy) || !aligned16(w->w_router) || !aligned16(w->w1) ||
        !aligned16(w->w2))
      return MOE_ERR_INVALID_ARG;
    if (!g->dx || !aligned16(g->dx) || !g->dw_router || !g->dw1 || !g->dw2 ||
        (w->b1 && !g->db1) || (w->b2 && !g->db2))
      return MOE_ERR_INVALID_ARG;
    if (S > 0 && (!w->shared_w1 || !w->shared_w2 || !aligned16(w->shared_w1) ||
                  !aligned16(w->shared_w2) || !g->dws1 || !g->dws2 ||
                  (w->shared_b1 && !g->dsb1) || (w->shared_b2 && !g->dsb2)))
      return MOE_ERR_INVALID_ARG;
  }
  st = ws_check(ws, ws_bytes, need);
  if (st != MOE_OK || ws == nullptr) return st;
  plan(ws, p);

  // combine and router backward (and the padded offsets of the
  // weight-gradient columns), then the router's weight and bias gradients
  if (p_terms)
    MOE_HIP_TRY(launch_aux_dp(c, sv->scores, sv->token_lse, sv->expert_counts, lw, p.aux_dp,
                              stream));
  CombineRouterBwd cb;
  cb.dy = dy;
  cb.y_perm = sv->y_perm;
  cb.inv_row = sv->inv_row;
  cb.topk_w = sv->topk_w;
  cb.d_yperm = p.dO;
  cb.scores = sv->scores;
  cb.lse = sv->token_lse;
  cb.topk_idx = sv->topk_idx;
  cb.counts = sv->expert_counts;
  cb.aux_dp = p_terms ? p.aux_dp : nullptr;
  cb.dl = p.dl;
  cb.offsets = sv->expert_offsets;
  cb.pad = kPad;
  cb.ncols = Rp;
  cb.poff = p.poff;
  cb.colrow = p.colrow;
  MOE_HIP_TRY(launch_combine_router_bwd(c, lw, cb, stream));
  const RouterWgradDesc rw{p.dl, x, T, E, d, nsplit, p.wr_part, g->dw_router, g->drouter_bias};

  // routed experts: transposed weights (with the router weight gradient's
  // split products in the same launch), dh, da / h (from the saved
  // pre-activations), dx rows
  TransposeDesc t2{w->w2, f, (int64_t)d * f, nullptr, nullptr, d, d, f, p.W2t, d,
                   (int64_t)f * d, E};
  TransposeDesc t1{w->w1, d, (int64_t)w1r * d, nullptr, nullptr, w1r, w1r, d, p.W1t, w1r,
                   (int64_t)d * w1r, E};
  MOE_HIP_TRY(launch_side(t2, t1, &rw, nullptr, stream));
  GemmDesc gd{};
  gd.group_off = sv->expert_offsets;
  gd.n_groups = E;
  gd.n_seg = 1;
  gd.rows_max = R;
  gd.a = p.dO;
  gd.a_rows = nullptr;
  gd.lda = d;
  gd.w = p.W2t;
  gd.bias = nullptr;
  gd.d = f;
  gd.f = d;
  gd.out = p.dH;
  gd.ldo = f;
  MOE_HIP_TRY(launch_gemm(c, kGemmDown, gd, stream));
  // da (row-major) and the expert-padded da^T, h^T in one pass
  MOE_HIP_TRY(launch_act_bwd_t(sv->preact, w1r, p.dH, f, p.colrow, 0, Rp, 1, f, c.act, p.dA, p.dAt,
                               p.Ht, Rp, stream));
  gd.a = p.dA;
  gd.lda = w1r;
  gd.w = p.W1t;
  gd.d = d;
  gd.f = w1r;
  gd.out = p.dXr;
  gd.ldo = d;
  MOE_HIP_TRY(launch_gemm(c, kGemmDown, gd, stream));

  // weight gradients from the expert-padded transposes of d o and x (the
  // router weight gradient's split sums in the same launch)
  TransposeDesc to{p.dO, d, 0, p.colrow, nullptr, 0, Rp, d, p.dOt, Rp, 0, 1};
  TransposeDesc tx{x, d, 0, p.colrow, sv->perm_token, 0, Rp, d, p.Xt, Rp, 0, 1};
  MOE_HIP_TRY(launch_side(to, tx, nullptr, &rw, stream));
  MOE_HIP_TRY(launch_wgrad(p.dOt, Rp, 0, p.Ht, Rp, 0, p.poff, Rp, d, f, E, g->dw2, f,
                           (int64_t)d * f, p.wg_part, stream));
  MOE_HIP_TRY(launch_wgrad(p.dAt, Rp, 0, p.Xt, Rp, 0, p.poff, Rp, w1r, d, E, g->dw1, d,
                           (int64_t)w1r * d, p.wg_part, stream));
  if (w->b2) MOE_HIP_TRY(launch_seg_rowsum(p.dOt, Rp, d, p.poff, Rp, E, g->db2, d, stream));
  if (w->b1) MOE_HIP_TRY(launch_seg_rowsum(p.dAt, Rp, w1r, p.poff, Rp, E, g->db1, w1r, stream));

  // shared experts: every token, d o = dy
  if (S > 0) {
    GemmDesc sd{};
    sd.group_off = nullptr;  // one dense group of T rows
    sd.n_groups = 1;
    sd.n_seg = 1;
    sd.rows_max = T;
    TransposeDesc s2{w->shared_w2, f, (int64_t)d * f, nullptr, nullptr, d, d, f, p.Ws2t, d,
                     (int64_t)f * d, S};
    TransposeDesc s1{w->shared_w1, d, (int64_t)w1r * d, nullptr, nullptr, w1r, w1r, d, p.Ws1t,
                     w1r, (int64_t)d * w1r, S};
    MOE_HIP_TRY(launch_transpose(s2, s1, stream));
    for (int s = 0; s < S; ++s) {
      sd.a = dy;
      sd.lda = d;
      sd.w = static_cast<const uint16_t*>(p.Ws2t) + (int64_t)s * f * d;
      sd.bias = nullptr;
      sd.d = f;
      sd.f = d;
      sd.out = static_cast<uint16_t*>(p.dHs) + (int64_t)s * f;
      sd.ldo = (int64_t)S * f;
      MOE_HIP_TRY(launch_gemm(c, kGemmDown, sd, stream));
    }
    MOE_HIP_TRY(launch_act_bwd_t(sv->shared_preact, (int64_t)S * w1r, p.dHs, (int64_t)S * f, nullptr,
                                 T, Tp, S, f, c.act, p.dAs, p.dAst, p.Hst, Tp, stream));
    sd.a = p.dAs;
    sd.lda = (int64_t)S * w1r;
    sd.n_seg = S;
    sd.w = p.Ws1t;
    sd.d = d;
    sd.f = w1r;
    sd.out = p.dXs;
    sd.ldo = d;
    MOE_HIP_TRY(launch_gemm(c, kGemmDown, sd, stream));
    TransposeDesc ty{dy, d, 0, nullptr, nullptr, T, Tp, d, p.dyt, Tp, 0, 1};
    TransposeDesc txs{x, d, 0, nullptr, nullptr, T, Tp, d, p.xt, Tp, 0, 1};
    MOE_HIP_TRY(launch_transpose(ty, txs, stream));
    MOE_HIP_TRY(launch_wgrad(p.dyt, Tp, 0, p.Hst, Tp, (int64_t)f * Tp, nullptr, Tp, d, f, S, g->dws2,
                             f, (int64_t)d * f, p.wg_part, stream));
    MOE_HIP_TRY(launch_wgrad(p.dAst, Tp, (int64_t)w1r * Tp, p.xt, Tp, 0, nullptr, Tp, w1r, d, S,
                             g->dws1, d, (int64_t)w1r * d, p.wg_part, stream));
    if (w->shared_b2)
      for (int s = 0; s < S; ++s)
        MOE_HIP_TRY(launch_seg_rowsum(p.dyt, Tp, d, nullptr, Tp, 1, g->dsb2 + (int64_t)s * d, d,
                                      stream));
    if (w->shared_b1)
      MOE_HIP_TRY(launch_seg_rowsum(p.dAst, Tp, S * w1r, nullptr, Tp, 1, g->dsb1, S * w1r, stream));
  }

  // dx: router product, kept expert rows, shared experts, residual
  MOE_HIP_TRY(launch_dx_final(c, p.dl, w->w_router, p.dXr, sv->inv_row, S > 0 ? p.dXs : nullptr,
                              c.add_residual ? dy : nullptr, g->dx, stream));
  return MOE_OK;
}

}  // extern "C"
