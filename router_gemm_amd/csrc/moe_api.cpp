// moe_api.cpp -- the C ABI declared in include/moe.h: host-side argument
// validation (everything is checked before anything is launched), workspace
// carving, and the launch sequence of each call.  No allocation, no host
// synchronisation, no device state kept between calls.

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/moe.h"
#include "../../include/moe_timing.h"
#include "moe_kernels.h"

namespace {

thread_local std::string g_last_error;

moe_status fail(moe_status s, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

moe_status hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return MOE_OK;
  return fail(MOE_EHIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
constexpr int kMaxK = 32;
constexpr int kMaxE = 1024;
// The expert kernels stage 2 x K/128 weight-block scales per work item in
// LDS, sized for K <= 16384 (K = H for gate/up, I or shared I for down).
constexpr int kMaxH = 16384;
constexpr int kMaxI = 16384;

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Activations and h are e4m3 + 1x128 scales for fp8 and MX FP4 experts.
bool is_fp8(const moe_layer *L) { return L->expert_dtype == MOE_FP8_E4M3FN || L->expert_dtype == MOE_MXFP4_E2M1; }
bool is_mx(const moe_layer *L) { return L->expert_dtype == MOE_MXFP4_E2M1; }
size_t esz(const moe_layer *L) { return is_fp8(L) ? 1 : 2; }

// Sequential carving of the caller's workspace.
struct Carve {
  char *base;
  size_t used = 0;
  explicit Carve(void *b) : base(static_cast<char *>(b)) {}
  template <class T>
  T *take(size_t count) {
    const size_t off = moe::align_up(used, kAlign);
    used = off + moe::align_up(count * sizeof(T), kAlign);
    return base ? reinterpret_cast<T *>(base + off) : nullptr;
  }
};

// ---------------------------------------------------------------- validation

moe_status check_layer_shape(const moe_layer *L, bool need_router) {
  if (!L) return fail(MOE_EINVAL, "layer is NULL");
  if (L->hidden <= 0 || L->inter <= 0 || L->num_experts <= 0 || L->shared_inter < 0)
    return fail(MOE_EINVAL, "bad layer dimensions H=%d I=%d E=%d Is=%d", L->hidden, L->inter,
                L->num_experts, L->shared_inter);
  if (L->expert_dtype != MOE_BF16 && L->expert_dtype != MOE_FP8_E4M3FN && L->expert_dtype != MOE_MXFP4_E2M1)
    return fail(MOE_EUNSUPPORTED, "expert_dtype %d is not MOE_BF16, MOE_FP8_E4M3FN or MOE_MXFP4_E2M1",
                L->expert_dtype);
  if (L->hidden % 128 != 0 || L->hidden > kMaxH)
    return fail(MOE_EUNSUPPORTED, "hidden %d must be a multiple of 128 and <= %d", L->hidden, kMaxH);
  if (L->num_experts > kMaxE) return fail(MOE_EUNSUPPORTED, "num_experts %d > %d", L->num_experts, kMaxE);
  if (L->inter > kMaxI || L->shared_inter > kMaxI)
    return fail(MOE_EUNSUPPORTED, "inter %d / shared_inter %d > %d", L->inter, L->shared_inter, kMaxI);
  if (is_fp8(L) && L->inter % 128 != 0)
    return fail(MOE_EUNSUPPORTED, "fp8 and mxfp4 experts need inter %% 128 == 0 (inter=%d)", L->inter);
  if (!is_fp8(L) && L->inter % 64 != 0)
    return fail(MOE_EUNSUPPORTED, "bf16 experts need inter %% 64 == 0 (inter=%d)", L->inter);
  if (L->shared_inter % 64 != 0)
    return fail(MOE_EUNSUPPORTED, "shared_inter %% 64 != 0 (%d)", L->shared_inter);
  if (need_router && (L->top_k < 1 || L->top_k > kMaxK || L->top_k > L->num_experts))
    return fail(MOE_EINVAL, "top_k %d outside [1, min(E=%d, %d)]", L->top_k, L->num_experts, kMaxK);
  if (L->top_k < 0 || L->top_k > kMaxK) return fail(MOE_EINVAL, "top_k %d outside [0, %d]", L->top_k, kMaxK);
  if (L->weight_layout != MOE_LAYOUT_ROWS && L->weight_layout != MOE_LAYOUT_TILE16)
    return fail(MOE_EINVAL, "weight_layout %d is not MOE_LAYOUT_ROWS or MOE_LAYOUT_TILE16", L->weight_layout);
  if (L->weight_layout == MOE_LAYOUT_TILE16 && is_mx(L))
    return fail(MOE_EUNSUPPORTED, "mxfp4 experts take row-major weights only");
  return MOE_OK;
}

moe_status check_expert_weights(const moe_layer *L) {
  if (!L->w_gate_up || !L->w_down) return fail(MOE_EINVAL, "expert weights are NULL");
  if (!aligned16(L->w_gate_up) || !aligned16(L->w_down)) return fail(MOE_EINVAL, "expert weights not 16-byte aligned");
  if (is_fp8(L) && (!L->s_gate_up || !L->s_down))
    return fail(MOE_EINVAL, "fp8 and mxfp4 experts need s_gate_up and s_down");
  if (is_mx(L) && (!aligned16(L->s_gate_up) || !aligned16(L->s_down)))
    return fail(MOE_EINVAL, "mxfp4 scale tensors not 16-byte aligned");
  return MOE_OK;
}

moe_status check_shared(const moe_layer *L) {
  if (L->shared_inter == 0) return MOE_OK;
  if (!L->w_shared_gate_up || !L->w_shared_down) return fail(MOE_EINVAL, "shared expert weights are NULL");
  if (!aligned16(L->w_shared_gate_up) || !aligned16(L->w_shared_down))
    return fail(MOE_EINVAL, "shared expert weights not 16-byte aligned");
  return MOE_OK;
}

moe_status check_rows(int64_t T, int64_t N) {
  if (T < 0 || N < 0) return fail(MOE_EINVAL, "negative size T=%lld N=%lld", (long long)T, (long long)N);
  if (T > (int64_t)INT32_MAX / 2 || N > (int64_t)INT32_MAX / 2)
    return fail(MOE_EINVAL, "size too large T=%lld N=%lld", (long long)T, (long long)N);
  return MOE_OK;
}

moe_status check_ws(const void *ws, size_t ws_bytes, size_t need) {
  if (need > ws_bytes)
    return fail(MOE_EWORKSPACE, "workspace of %zu bytes, need %zu", ws_bytes, need);
  if (need > 0 && !ws) return fail(MOE_EINVAL, "workspace is NULL");
  if (((uintptr_t)ws & (kAlign - 1)) != 0) return fail(MOE_EINVAL, "workspace not %zu-byte aligned", kAlign);
  return MOE_OK;
}

bool out_dtype_ok(int32_t d) { return d == MOE_BF16 || d == MOE_F32; }

// ---------------------------------------------------------------- workspace plans

struct RouteWs {
  float *partial;
  int S;
};
RouteWs carve_route(Carve &c, const moe_layer *L, int64_t T) {
  RouteWs r;
  r.S = moe::router_ksplit(T, L->num_experts, L->hidden);
  r.partial = c.take<float>((size_t)r.S * T * L->num_experts + 1);
  return r;
}

int32_t *carve_sort(Carve &c, int64_t N, int64_t nbins) { return c.take<int32_t>(moe::sort_ws_words(N, nbins) + 1); }

// Expert-FFN workspace: the tile list plus each group's intermediate h.
struct FfnWs {
  moe::FfnPlan plan;
  int32_t *tiles;
  uint8_t *h[moe::kMaxGroups];
  float *hs[moe::kMaxGroups];
};
FfnWs carve_ffn(Carve &c, moe::FfnGroup *g, int ngroups, int H) {
  FfnWs f;
  f.plan = moe::ffn_plan(g, ngroups, H);
  f.tiles = c.take<int32_t>(moe::ffn_tiles_bytes(f.plan) / 4);
  for (int i = 0; i < ngroups; ++i) {
    f.h[i] = c.take<uint8_t>((size_t)g[i].nrows * g[i].I * (g[i].fp8 ? 1 : 2) + 16);
    f.hs[i] = g[i].fp8 ? c.take<float>((size_t)g[i].nrows * (g[i].I / 128) + 1) : nullptr;
    g[i].h = f.h[i];
    g[i].hs = f.hs[i];
  }
  return f;
}

moe::FfnGroup routed_group(const moe_layer *L, const void *x_perm, const float *x_scale, const int32_t *off,
                           int64_t N, void *y, bool y_f32) {
  moe::FfnGroup g{};
  g.x = static_cast<const uint8_t *>(x_perm);
  g.xs = x_scale;
  g.wgu = static_cast<const uint8_t *>(L->w_gate_up);
  g.wd = static_cast<const uint8_t *>(L->w_down);
  if (is_mx(L)) {
    g.mgu = static_cast<const uint8_t *>(L->s_gate_up);
    g.md = static_cast<const uint8_t *>(L->s_down);
  } else {
    g.sgu = static_cast<const float *>(L->s_gate_up);
    g.sd = static_cast<const float *>(L->s_down);
  }
  g.off = off;
  g.y = y;
  g.E = L->num_experts;
  g.I = L->inter;
  g.nrows = (int32_t)N;
  g.fp8 = is_fp8(L) ? 1 : 0;
  g.mx = is_mx(L) ? 1 : 0;
  g.y_f32 = y_f32 ? 1 : 0;
  g.tile16 = L->weight_layout == MOE_LAYOUT_TILE16 ? 1 : 0;
  return g;
}

moe::FfnGroup shared_group(const moe_layer *L, const void *x, const int32_t *off2, int64_t T, void *y, bool y_f32) {
  moe::FfnGroup g{};
  g.x = static_cast<const uint8_t *>(x);
  g.wgu = static_cast<const uint8_t *>(L->w_shared_gate_up);
  g.wd = static_cast<const uint8_t *>(L->w_shared_down);
  g.off = off2;
  g.y = y;
  g.E = 1;
  g.I = L->shared_inter;
  g.nrows = (int32_t)T;
  g.fp8 = 0;
  g.y_f32 = y_f32 ? 1 : 0;
  return g;
}

struct CombineWs {
  int32_t *tok_off, *tok_list, *sort;
};
CombineWs carve_combine(Carve &c, int64_t T, int64_t N) {
  CombineWs w;
  w.tok_off = c.take<int32_t>((size_t)T + 1);
  w.tok_list = c.take<int32_t>((size_t)N + 1);
  w.sort = carve_sort(c, N, T);
  return w;
}

struct ForwardWs {
  int32_t *ids;
  float *gates;
  RouteWs route;
  int32_t *offsets, *perm_src, *perm_pos, *sort;
  uint8_t *x_perm;
  float *x_scale;
  FfnWs ffn;                       // routed (+ shared) experts in one launch
  moe::FfnGroup groups[moe::kMaxGroups];
  int ngroups;
  // A shared expert whose width is not a multiple of 128 next to routed
  // experts whose width is: its own launch (streaming kernels), so that the
  // routed experts keep the 128-column kernels (LDS-tiled, or fp8).
  bool shared_apart;
  FfnWs ffn_sh;
  moe::FfnGroup sh_group;
  uint16_t *y_perm;
  void *sh_out;
};
ForwardWs carve_forward(Carve &c, const moe_layer *L, const void *x, int64_t T, bool out_f32) {
  ForwardWs f;
  const int64_t N = T * L->top_k;
  const int H = L->hidden, E = L->num_experts;
  f.ids = c.take<int32_t>((size_t)N + 1);
  f.gates = c.take<float>((size_t)N + 1);
  f.route = carve_route(c, L, T);
  f.offsets = c.take<int32_t>((size_t)E + 1);
  f.perm_src = c.take<int32_t>((size_t)N + 1);
  f.perm_pos = c.take<int32_t>((size_t)N + 1);
  f.sort = carve_sort(c, N, E);
  f.x_perm = c.take<uint8_t>((size_t)N * H * esz(L) + 16);
  f.x_scale = is_fp8(L) ? c.take<float>((size_t)N * (H / 128) + 1) : nullptr;
  f.y_perm = c.take<uint16_t>((size_t)N * H + 8);
  f.ngroups = 0;
  f.shared_apart = L->shared_inter > 0 && L->shared_inter % 128 != 0 && L->inter % 128 == 0;
  if (L->shared_inter > 0) {
    f.sh_out = c.take<uint8_t>((size_t)T * H * (out_f32 ? 4 : 2) + 16);
    // the shared expert's tiles go first in the list: they carry twice the bytes
    // (bf16); no offsets array: one expert holding all T rows
    if (!f.shared_apart) f.groups[f.ngroups++] = shared_group(L, x, nullptr, T, f.sh_out, out_f32);
  } else {
    f.sh_out = nullptr;
  }
  f.groups[f.ngroups++] = routed_group(L, f.x_perm, f.x_scale, f.offsets, N, f.y_perm, false);
  f.ffn = carve_ffn(c, f.groups, f.ngroups, H);
  if (f.shared_apart) {
    f.sh_group = shared_group(L, x, nullptr, T, f.sh_out, out_f32);
    f.ffn_sh = carve_ffn(c, &f.sh_group, 1, H);
  }
  return f;
}

// Forward for pre-routed assignments: the grouping, the gathered (and, fp8,
// quantised) rows, routed + shared expert FFN, and the per-token grouping of
// the combine.
struct RoutedWs {
  int32_t *offsets, *perm_src, *perm_pos, *sort;
  uint8_t *x_perm;
  float *x_scale;
  FfnWs ffn;
  moe::FfnGroup groups[moe::kMaxGroups];
  int ngroups;
  bool shared_apart;
  FfnWs ffn_sh;
  moe::FfnGroup sh_group;
  uint16_t *y_perm;
  void *sh_out;
  CombineWs comb;
};
RoutedWs carve_routed(Carve &c, const moe_layer *L, const void *x, int64_t T, int64_t N, bool out_f32) {
  RoutedWs f;
  const int H = L->hidden, E = L->num_experts;
  f.offsets = c.take<int32_t>((size_t)E + 1);
  f.perm_src = c.take<int32_t>((size_t)N + 1);
  f.perm_pos = c.take<int32_t>((size_t)N + 1);
  f.sort = carve_sort(c, N, E);
  f.x_perm = c.take<uint8_t>((size_t)N * H * esz(L) + 16);
  f.x_scale = is_fp8(L) ? c.take<float>((size_t)N * (H / 128) + 1) : nullptr;
  f.y_perm = c.take<uint16_t>((size_t)N * H + 8);
  f.ngroups = 0;
  f.shared_apart = L->shared_inter > 0 && L->shared_inter % 128 != 0 && L->inter % 128 == 0;
  f.sh_out = nullptr;
  if (L->shared_inter > 0) {
    f.sh_out = c.take<uint8_t>((size_t)T * H * (out_f32 ? 4 : 2) + 16);
    if (!f.shared_apart) f.groups[f.ngroups++] = shared_group(L, x, nullptr, T, f.sh_out, out_f32);
  }
  f.groups[f.ngroups++] = routed_group(L, f.x_perm, f.x_scale, f.offsets, N, f.y_perm, false);
  f.ffn = carve_ffn(c, f.groups, f.ngroups, H);
  if (f.shared_apart) {
    f.sh_group = shared_group(L, x, nullptr, T, f.sh_out, out_f32);
    f.ffn_sh = carve_ffn(c, &f.sh_group, 1, H);
  }
  f.comb = carve_combine(c, T, N);
  return f;
}

// Backward: the sort, rows gathered into expert order, and each expert set's
// scratch (routed experts; shared expert).
struct BackwardWs {
  int32_t *offsets, *perm_src, *perm_pos, *sort;
  uint16_t *x_perm, *dy_perm;
  float *dl;
  moe::BwdExpert routed, shared;
};
void carve_bwd_expert(Carve &c, moe::BwdExpert &X, int H, int I, int G, int64_t rows, bool with_dg) {
  X = moe::BwdExpert{};
  X.H = H;
  X.I = I;
  X.G = G;
  X.rows = rows;
  X.z = c.take<float>((size_t)rows * 2 * I + 1);
  X.u = c.take<float>((size_t)rows * I + 1);
  X.hg = c.take<uint16_t>((size_t)rows * I + 8);
  X.dz = c.take<uint16_t>((size_t)rows * 2 * I + 8);
  X.dg = with_dg ? c.take<float>((size_t)rows + 1) : nullptr;
  X.dx_rows = c.take<float>((size_t)rows * H + 1);
  X.max_tiles = moe::bwd_max_tiles(rows, G);
  X.tiles = c.take<int32_t>((size_t)moe::kTileHdrWords + 2 * (size_t)X.max_tiles);
}
BackwardWs carve_backward(Carve &c, const moe_layer *L, int64_t T) {
  BackwardWs b;
  const int64_t N = T * L->top_k;
  const int H = L->hidden, E = L->num_experts;
  b.offsets = c.take<int32_t>((size_t)E + 1);
  b.perm_src = c.take<int32_t>((size_t)N + 1);
  b.perm_pos = c.take<int32_t>((size_t)N + 1);
  b.sort = carve_sort(c, N, E);
  b.x_perm = c.take<uint16_t>((size_t)N * H + 8);
  b.dy_perm = c.take<uint16_t>((size_t)N * H + 8);
  b.dl = c.take<float>((size_t)N + 1);
  carve_bwd_expert(c, b.routed, H, L->inter, E, N, true);
  if (L->shared_inter > 0) carve_bwd_expert(c, b.shared, H, L->shared_inter, 1, T, false);
  return b;
}
size_t need_backward(const moe_layer *L, int64_t T) {
  Carve c(nullptr);
  carve_backward(c, L, T);
  return c.used;
}

size_t need_route(const moe_layer *L, int64_t T) { Carve c(nullptr); carve_route(c, L, T); return c.used; }
size_t need_permute(const moe_layer *L, int64_t N) { Carve c(nullptr); carve_sort(c, N, L->num_experts); return c.used; }
size_t need_ffn(const moe_layer *L, int64_t N) {
  Carve c(nullptr);
  moe::FfnGroup g = routed_group(L, nullptr, nullptr, nullptr, N, nullptr, false);
  carve_ffn(c, &g, 1, L->hidden);
  return c.used;
}
size_t need_combine(int64_t T, int64_t N, bool tokens) {
  if (!tokens) return 0;
  Carve c(nullptr);
  carve_combine(c, T, N);
  return c.used;
}
size_t need_forward(const moe_layer *L, int64_t T) {
  Carve c(nullptr);
  carve_forward(c, L, nullptr, T, true);
  return c.used;
}
size_t need_routed(const moe_layer *L, int64_t T, int64_t N) {
  Carve c(nullptr);
  carve_routed(c, L, nullptr, T, N, true);
  return c.used;
}

}  // namespace

extern "C" {

const char *moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_EINVAL: return "MOE_EINVAL: invalid argument";
    case MOE_EUNSUPPORTED: return "MOE_EUNSUPPORTED: configuration not built";
    case MOE_EWORKSPACE: return "MOE_EWORKSPACE: workspace too small";
    case MOE_EHIP: return "MOE_EHIP: HIP launch failed";
  }
  return "unknown moe_status";
}

const char *moe_last_error(void) { return g_last_error.c_str(); }

size_t moe_workspace_bytes(const moe_layer *L, int64_t T, int64_t N) {
  if (check_layer_shape(L, false) != MOE_OK || check_rows(T, N) != MOE_OK) return 0;
  size_t need = 0;
  auto upd = [&](size_t v) { need = v > need ? v : need; };
  upd(need_permute(L, N));
  upd(need_ffn(L, N));
  upd(need_combine(T, N, true));
  upd(need_routed(L, T, N));
  if (L->top_k >= 1) {
    upd(need_route(L, T));
    upd(need_forward(L, T));
  }
  return need;
}

moe_status moe_route(const moe_layer *L, const void *x, int64_t T, int32_t *topk_ids, float *topk_gates,
                     float *logits, void *ws, size_t ws_bytes, void *stream) {
  moe_status s;
  if ((s = check_layer_shape(L, true)) != MOE_OK) return s;
  if ((s = check_rows(T, 0)) != MOE_OK) return s;
  if (T > 0) {
    if (!L->w_router || !x || !topk_ids || !topk_gates) return fail(MOE_EINVAL, "NULL router argument");
    if (!aligned16(x) || !aligned16(L->w_router)) return fail(MOE_EINVAL, "x or w_router not 16-byte aligned");
  }
  if (T == 0) return MOE_OK;
  if ((s = check_ws(ws, ws_bytes, need_route(L, T))) != MOE_OK) return s;
  Carve c(ws);
  RouteWs r = carve_route(c, L, T);
  return hip_status(moe::launch_router(static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(L->w_router),
                                       L->router_bias, T, L->num_experts, L->hidden, L->top_k, r.partial, r.S,
                                       topk_ids, topk_gates, logits, (hipStream_t)stream),
                    "moe_route");
}

moe_status moe_permute(const moe_layer *L, const void *x, int64_t T, const int32_t *assign_expert,
                       const int32_t *assign_token, int64_t N, int32_t *expert_offsets, int32_t *perm_src,
                       int32_t *perm_pos, void *x_perm, float *x_scale, void *ws, size_t ws_bytes,
                       void *stream) {
  moe_status s;
  if ((s = check_layer_shape(L, false)) != MOE_OK) return s;
  if ((s = check_rows(T, N)) != MOE_OK) return s;
  if (!assign_token) {
    if (L->top_k < 1) return fail(MOE_EINVAL, "assign_token is NULL but top_k < 1");
    if (N != T * L->top_k) return fail(MOE_EINVAL, "N=%lld != T*k=%lld without assign_token", (long long)N,
                                       (long long)(T * L->top_k));
  }
  if (!expert_offsets) return fail(MOE_EINVAL, "expert_offsets is NULL");
  if (N > 0) {
    if (!x || !assign_expert || !perm_src || !perm_pos || !x_perm) return fail(MOE_EINVAL, "NULL permute argument");
    if (is_fp8(L) && !x_scale) return fail(MOE_EINVAL, "fp8 experts need x_scale");
    if (!aligned16(x) || !aligned16(x_perm)) return fail(MOE_EINVAL, "x or x_perm not 16-byte aligned");
  }
  if ((s = check_ws(ws, ws_bytes, need_permute(L, N))) != MOE_OK) return s;
  hipStream_t st = (hipStream_t)stream;  // N == 0 still writes expert_offsets (all zero)
  Carve c(ws);
  int32_t *sort = carve_sort(c, N, L->num_experts);
  hipError_t e = moe::launch_counting_sort(assign_expert, assign_token, T, N, L->num_experts, expert_offsets,
                                           perm_src, perm_pos, sort, st);
  if (e != hipSuccess) return hip_status(e, "moe_permute: sort");
  e = moe::launch_gather_rows(static_cast<const uint16_t *>(x), L->hidden, perm_src, assign_token, L->top_k, N,
                              expert_offsets + L->num_experts, is_fp8(L), x_perm, x_scale, st);
  return hip_status(e, "moe_permute: gather");
}

moe_status moe_expert_ffn(const moe_layer *L, const int32_t *expert_offsets, const void *x_perm,
                          const float *x_scale, int64_t N, void *y_perm, int32_t y_dtype, void *ws,
                          size_t ws_bytes, void *stream) {
  moe_status s;
  if ((s = check_layer_shape(L, false)) != MOE_OK) return s;
  if ((s = check_rows(0, N)) != MOE_OK) return s;
  if (!out_dtype_ok(y_dtype)) return fail(MOE_EUNSUPPORTED, "y_dtype %d is not MOE_BF16 or MOE_F32", y_dtype);
  if (N > 0) {
    if ((s = check_expert_weights(L)) != MOE_OK) return s;
    if (!expert_offsets || !x_perm || !y_perm) return fail(MOE_EINVAL, "NULL expert_ffn argument");
    if (is_fp8(L) && !x_scale) return fail(MOE_EINVAL, "fp8 experts need x_scale");
    if (!aligned16(x_perm) || !aligned16(y_perm)) return fail(MOE_EINVAL, "x_perm or y_perm not 16-byte aligned");
  }
  if (N == 0) return MOE_OK;
  if ((s = check_ws(ws, ws_bytes, need_ffn(L, N))) != MOE_OK) return s;
  Carve c(ws);
  moe::FfnGroup g = routed_group(L, x_perm, x_scale, expert_offsets, N, y_perm, y_dtype == MOE_F32);
  FfnWs f = carve_ffn(c, &g, 1, L->hidden);
  return hip_status(moe::launch_expert_ffn(&g, 1, L->hidden, f.plan, f.tiles, MOE_SITE_GATE_UP, (hipStream_t)stream),
                    "moe_expert_ffn");
}

moe_status moe_combine(const moe_layer *L, const void *y_perm, int32_t y_dtype, const int32_t *perm_pos,
                       const int32_t *assign_token, const float *gates, int64_t N, const void *shared_out,
                       int32_t shared_dtype, int64_t T, void *y, int32_t out_dtype, void *ws, size_t ws_bytes,
                       void *stream) {
  moe_status s;
  if ((s = check_layer_shape(L, false)) != MOE_OK) return s;
  if ((s = check_rows(T, N)) != MOE_OK) return s;
  if (!out_dtype_ok(y_dtype) || !out_dtype_ok(out_dtype) || (shared_out && !out_dtype_ok(shared_dtype)))
    return fail(MOE_EUNSUPPORTED, "dtypes must be MOE_BF16 or MOE_F32");
  if (!assign_token) {
    if (L->top_k < 1) return fail(MOE_EINVAL, "assign_token is NULL but top_k < 1");
    if (N != T * L->top_k) return fail(MOE_EINVAL, "N=%lld != T*k without assign_token", (long long)N);
  }
  if (T > 0) {
    if (!y || !aligned16(y)) return fail(MOE_EINVAL, "y NULL or not 16-byte aligned");
    if (shared_out && !aligned16(shared_out)) return fail(MOE_EINVAL, "shared_out not 16-byte aligned");
  }
  if (N > 0 && (!y_perm || !perm_pos || !gates || !aligned16(y_perm)))
    return fail(MOE_EINVAL, "NULL or misaligned combine argument");
  if (T == 0) return MOE_OK;
  if ((s = check_ws(ws, ws_bytes, need_combine(T, N, assign_token != nullptr))) != MOE_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  const int32_t *tok_off = nullptr, *tok_list = nullptr;
  if (assign_token) {
    Carve c(ws);
    CombineWs w = carve_combine(c, T, N);
    hipError_t e = moe::launch_counting_sort(assign_token, nullptr, 0, N, T, w.tok_off, w.tok_list, nullptr,
                                             w.sort, st);
    if (e != hipSuccess) return hip_status(e, "moe_combine: token sort");
    tok_off = w.tok_off;
    tok_list = w.tok_list;
  }
  return hip_status(moe::launch_combine(y_perm, y_dtype == MOE_F32, perm_pos, tok_off, tok_list, L->top_k, gates,
                                        shared_out, shared_dtype == MOE_F32, T, L->hidden, N, y, out_dtype == MOE_F32, st),
                    "moe_combine");
}

namespace {
// The expert GEMMs' tile list, for the sort to write from its own offsets (the
// shared expert's group first when it rides in the routed launches); none for
// MX layers on 64-row tiles, whose groups get lists of their own.
moe::SmallTiles sort_tiles(const moe_layer *L, const FfnWs &ffn, int ngroups, int64_t T) {
  if (ffn.plan.tiled && is_mx(L) && ffn.plan.bm != 256) return moe::SmallTiles{};
  return moe::SmallTiles{reinterpret_cast<moe::TileEntry *>(ffn.tiles + moe::kTileHdrWords), ffn.tiles, ffn.plan.bm,
                         ffn.plan.max_tiles, ngroups == 2 ? 1 : 0, (int)T};
}

moe_status forward_impl(const moe_layer *L, const void *x, int64_t T, void *y, int32_t out_dtype, int32_t *topk_ids,
                        float *topk_gates, float *z_saved, void *ws, size_t ws_bytes, void *stream) {
  moe_status s;
  if ((s = check_layer_shape(L, true)) != MOE_OK) return s;
  if ((s = check_rows(T, T * (int64_t)L->top_k)) != MOE_OK) return s;
  if (!out_dtype_ok(out_dtype)) return fail(MOE_EUNSUPPORTED, "out_dtype %d is not MOE_BF16 or MOE_F32", out_dtype);
  if (T > 0) {
    if (!x || !y || !L->w_router) return fail(MOE_EINVAL, "NULL forward argument");
    if (!aligned16(x) || !aligned16(y) || !aligned16(L->w_router)) return fail(MOE_EINVAL, "x, y or w_router not 16-byte aligned");
    if ((s = check_expert_weights(L)) != MOE_OK) return s;
    if ((s = check_shared(L)) != MOE_OK) return s;
  }
  if (T == 0) return MOE_OK;
  if ((s = check_ws(ws, ws_bytes, need_forward(L, T))) != MOE_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  const bool out_f32 = out_dtype == MOE_F32;
  const int64_t N = T * L->top_k;
  const int H = L->hidden, E = L->num_experts;
  Carve c(ws);
  ForwardWs f = carve_forward(c, L, x, T, out_f32);
  int32_t *ids = topk_ids ? topk_ids : f.ids;
  float *gates = topk_gates ? topk_gates : f.gates;
  hipError_t e;
  e = moe::launch_router(static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(L->w_router), L->router_bias,
                         T, E, H, L->top_k, f.route.partial, f.route.S, ids, gates, nullptr, st);
  if (e != hipSuccess) return hip_status(e, "moe_forward: route");
  moe::FfnGroup &R = f.groups[f.ngroups - 1];
  bool tiles_ready = false;
  if (!f.ffn.plan.tiled && moe::permute_small_ok(N, E)) {
    // a decode-sized call: sort, tables, tile list and row gather in one launch
    moe::SmallTiles tl{reinterpret_cast<moe::TileEntry *>(f.ffn.tiles + moe::kTileHdrWords), f.ffn.tiles,
                       f.ffn.plan.bm, f.ffn.plan.max_tiles, f.ngroups == 2 ? 1 : 0, (int)T};
    e = moe::launch_permute_small(ids, N, E, L->top_k, static_cast<const uint16_t *>(x), H, is_fp8(L), f.offsets,
                                  f.perm_src, f.perm_pos, f.x_perm, f.x_scale, tl, st);
    if (e != hipSuccess) return hip_status(e, "moe_forward: grouping");
    tiles_ready = true;
  } else {
    e = moe::launch_counting_sort_tiles(ids, nullptr, 0, N, E, f.offsets, f.perm_src, f.perm_pos, f.sort,
                                        sort_tiles(L, f.ffn, f.ngroups, T), &tiles_ready, st);
    if (e != hipSuccess) return hip_status(e, "moe_forward: sort");
    // LDS-tiled expert kernels read the routed rows through the sort permutation
    // (x quantised once per token for fp8 experts) instead of a gathered copy;
    // their per-lane row offsets are 32-bit.
    if (f.ffn.plan.tiled && T * H * (int64_t)esz(L) < (int64_t(1) << 31)) {
      R.xsrc = f.perm_src;
      R.xdiv = L->top_k;
      if (is_fp8(L)) {
        e = moe::launch_quantize_rows(static_cast<const uint16_t *>(x), H, T, f.x_perm, f.x_scale, st);
        if (e != hipSuccess) return hip_status(e, "moe_forward: quantise");
      } else {
        R.x = static_cast<const uint8_t *>(x);
      }
    } else {
      e = moe::launch_gather_rows(static_cast<const uint16_t *>(x), H, f.perm_src, nullptr, L->top_k, N, f.offsets + E,
                                  is_fp8(L), f.x_perm, f.x_scale, st);
      if (e != hipSuccess) return hip_status(e, "moe_forward: gather");
    }
  }
  if (z_saved) {   // routed rows in expert order, then the shared expert's rows
    R.z = z_saved;
    if (f.ngroups == 2) f.groups[0].z = z_saved + (size_t)N * 2 * L->inter;
    if (f.shared_apart) f.sh_group.z = z_saved + (size_t)N * 2 * L->inter;
  }
  e = moe::launch_expert_ffn(f.groups, f.ngroups, H, f.ffn.plan, f.ffn.tiles, MOE_SITE_GATE_UP, st, tiles_ready);
  if (e != hipSuccess) return hip_status(e, "moe_forward: experts");
  if (f.shared_apart) {
    e = moe::launch_expert_ffn(&f.sh_group, 1, H, f.ffn_sh.plan, f.ffn_sh.tiles, MOE_SITE_GATE_UP, st);
    if (e != hipSuccess) return hip_status(e, "moe_forward: shared expert");
  }
  e = moe::launch_combine(f.y_perm, false, f.perm_pos, nullptr, nullptr, L->top_k, gates, f.sh_out, out_f32, T, H, N, y,
                          out_f32, st);
  return hip_status(e, "moe_forward: combine");
}
}  // namespace

moe_status moe_forward(const moe_layer *L, const void *x, int64_t T, void *y, int32_t out_dtype, int32_t *topk_ids,
                       float *topk_gates, void *ws, size_t ws_bytes, void *stream) {
  return forward_impl(L, x, T, y, out_dtype, topk_ids, topk_gates, nullptr, ws, ws_bytes, stream);
}

moe_status moe_forward_routed(const moe_layer *L, const void *x, int64_t T, const int32_t *assign_expert,
                              const int32_t *assign_token, const float *gates, int64_t N, void *y, int32_t out_dtype,
                              void *ws, size_t ws_bytes, void *stream) {
  moe_status s;
  if ((s = check_layer_shape(L, false)) != MOE_OK) return s;
  if ((s = check_rows(T, N)) != MOE_OK) return s;
  if (!out_dtype_ok(out_dtype)) return fail(MOE_EUNSUPPORTED, "out_dtype %d is not MOE_BF16 or MOE_F32", out_dtype);
  if (T > 0) {
    if (!x || !y) return fail(MOE_EINVAL, "NULL forward argument");
    if (!aligned16(x) || !aligned16(y)) return fail(MOE_EINVAL, "x or y not 16-byte aligned");
    if ((s = check_shared(L)) != MOE_OK) return s;
  }
  if (N > 0) {
    if (!assign_expert || !assign_token || !gates) return fail(MOE_EINVAL, "NULL assignment argument");
    if ((s = check_expert_weights(L)) != MOE_OK) return s;
  }
  if (T == 0) return MOE_OK;   // no token: every assignment is out of range, nothing to write
  if ((s = check_ws(ws, ws_bytes, need_routed(L, T, N))) != MOE_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  const bool out_f32 = out_dtype == MOE_F32;
  const int H = L->hidden, E = L->num_experts;
  Carve c(ws);
  RoutedWs f = carve_routed(c, L, x, T, N, out_f32);
  bool tiles_ready = false;
  hipError_t e = moe::launch_counting_sort_tiles(assign_expert, assign_token, T, N, E, f.offsets, f.perm_src,
                                                 f.perm_pos, f.sort, sort_tiles(L, f.ffn, f.ngroups, T), &tiles_ready,
                                                 st);
  if (e != hipSuccess) return hip_status(e, "moe_forward_routed: sort");
  e = moe::launch_gather_rows(static_cast<const uint16_t *>(x), H, f.perm_src, assign_token, 1, N, f.offsets + E,
                              is_fp8(L), f.x_perm, f.x_scale, st);
  if (e != hipSuccess) return hip_status(e, "moe_forward_routed: gather");
  // routed and shared expert in the same launches
  e = moe::launch_expert_ffn(f.groups, f.ngroups, H, f.ffn.plan, f.ffn.tiles, MOE_SITE_GATE_UP, st, tiles_ready);
  if (e != hipSuccess) return hip_status(e, "moe_forward_routed: experts");
  if (f.shared_apart) {
    e = moe::launch_expert_ffn(&f.sh_group, 1, H, f.ffn_sh.plan, f.ffn_sh.tiles, MOE_SITE_GATE_UP, st);
    if (e != hipSuccess) return hip_status(e, "moe_forward_routed: shared expert");
  }
  e = moe::launch_counting_sort(assign_token, nullptr, 0, N, T, f.comb.tok_off, f.comb.tok_list, nullptr,
                                f.comb.sort, st);
  if (e != hipSuccess) return hip_status(e, "moe_forward_routed: token sort");
  e = moe::launch_combine(f.y_perm, false, f.perm_pos, f.comb.tok_off, f.comb.tok_list, 0, gates, f.sh_out, out_f32, T,
                          H, N, y, out_f32, st);
  return hip_status(e, "moe_forward_routed: combine");
}

}  // extern "C"

namespace moe {
// For the variant of moe_forward whose scratch memory is the library's static
// device array (scratch.hip).
size_t forward_ws_bytes(const moe_layer *L, int64_t T) {
  if (check_layer_shape(L, true) != MOE_OK || check_rows(T, T * (int64_t)L->top_k) != MOE_OK) return 0;
  return need_forward(L, T);
}
moe_status forward_with_ws(const moe_layer *L, const void *x, int64_t T, void *y, int32_t out_dtype,
                           int32_t *topk_ids, float *topk_gates, void *ws, size_t ws_bytes, void *stream) {
  return forward_impl(L, x, T, y, out_dtype, topk_ids, topk_gates, nullptr, ws, ws_bytes, stream);
}
moe_status api_error(moe_status s, const char *msg) { return fail(s, "%s", msg); }
}  // namespace moe

extern "C" {

size_t moe_saved_z_floats(const moe_layer *L, int64_t T) {
  if (check_layer_shape(L, true) != MOE_OK || check_rows(T, T * (int64_t)L->top_k) != MOE_OK) return 0;
  return (size_t)T * L->top_k * 2 * L->inter + (size_t)T * 2 * L->shared_inter;
}

moe_status moe_forward_train(const moe_layer *L, const void *x, int64_t T, void *y, int32_t out_dtype,
                             int32_t *topk_ids, float *topk_gates, float *z_saved, void *ws, size_t ws_bytes,
                             void *stream) {
  moe_status s;
  if ((s = check_layer_shape(L, true)) != MOE_OK) return s;
  if (L->expert_dtype != MOE_BF16) return fail(MOE_EUNSUPPORTED, "moe_forward_train needs bf16 experts");
  if (L->weight_layout != MOE_LAYOUT_ROWS)
    return fail(MOE_EUNSUPPORTED, "moe_forward_train takes row-major expert weights");
  if (T > 0 && (!topk_ids || !topk_gates || !z_saved))
    return fail(MOE_EINVAL, "moe_forward_train needs topk_ids, topk_gates and z_saved");
  if (T > 0 && !aligned16(z_saved)) return fail(MOE_EINVAL, "z_saved not 16-byte aligned");
  return forward_impl(L, x, T, y, out_dtype, topk_ids, topk_gates, z_saved, ws, ws_bytes, stream);
}

size_t moe_backward_workspace_bytes(const moe_layer *L, int64_t T) {
  if (check_layer_shape(L, true) != MOE_OK || check_rows(T, T * (int64_t)L->top_k) != MOE_OK) return 0;
  return need_backward(L, T);
}

moe_status moe_backward(const moe_layer *L, const void *x, int64_t T, const int32_t *topk_ids,
                        const float *topk_gates, const void *dy, const float *z_saved, float *dx,
                        float *dw_gate_up, float *dw_down,
                        float *dw_shared_gate_up, float *dw_shared_down, float *dw_router, float *dbias, void *ws,
                        size_t ws_bytes, void *stream) {
  moe_status s;
  if ((s = check_layer_shape(L, true)) != MOE_OK) return s;
  if (L->expert_dtype != MOE_BF16) return fail(MOE_EUNSUPPORTED, "moe_backward needs bf16 experts");
  if (L->weight_layout != MOE_LAYOUT_ROWS)
    return fail(MOE_EUNSUPPORTED, "moe_backward takes row-major expert weights");
  if ((s = check_rows(T, T * (int64_t)L->top_k)) != MOE_OK) return s;
  if (T > 0) {
    if (!x || !dy || !topk_ids || !topk_gates || !L->w_router) return fail(MOE_EINVAL, "NULL backward input");
    if (!dx || !dw_gate_up || !dw_down || !dw_router) return fail(MOE_EINVAL, "NULL backward output");
    if (L->shared_inter > 0 && (!dw_shared_gate_up || !dw_shared_down))
      return fail(MOE_EINVAL, "shared expert gradients are NULL");
    if (!aligned16(x) || !aligned16(dy) || !aligned16(L->w_router)) return fail(MOE_EINVAL, "x, dy or w_router not 16-byte aligned");
    if (!aligned16(dx) || !aligned16(dw_gate_up) || !aligned16(dw_down) || !aligned16(dw_router) || !aligned16(z_saved) ||
        !aligned16(dw_shared_gate_up) || !aligned16(dw_shared_down))
      return fail(MOE_EINVAL, "gradient outputs not 16-byte aligned");
    if ((s = check_expert_weights(L)) != MOE_OK) return s;
    if ((s = check_shared(L)) != MOE_OK) return s;
  }
  if (T == 0) return MOE_OK;
  if ((s = check_ws(ws, ws_bytes, need_backward(L, T))) != MOE_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  const int64_t N = T * L->top_k;
  const int H = L->hidden, E = L->num_experts, k = L->top_k;
  Carve c(ws);
  BackwardWs b = carve_backward(c, L, T);
  hipError_t e = moe::launch_counting_sort(topk_ids, nullptr, 0, N, E, b.offsets, b.perm_src, b.perm_pos, b.sort, st);
  if (e != hipSuccess) return hip_status(e, "moe_backward: sort");
  e = moe::launch_gather_rows(static_cast<const uint16_t *>(x), H, b.perm_src, nullptr, k, N, b.offsets + E, false,
                              b.x_perm, nullptr, st);
  if (e != hipSuccess) return hip_status(e, "moe_backward: gather x");
  e = moe::launch_gather_rows(static_cast<const uint16_t *>(dy), H, b.perm_src, nullptr, k, N, b.offsets + E, false,
                              b.dy_perm, nullptr, st);
  if (e != hipSuccess) return hip_status(e, "moe_backward: gather dy");
  // routed experts: rows [0, offsets[E]) in expert order (rows beyond are
  // dropped assignments, outside every expert's range)
  moe::BwdExpert &R = b.routed;
  R.T = T;
  R.k = k;
  R.x = b.x_perm;
  R.dy = b.dy_perm;
  R.wgu = static_cast<const uint16_t *>(L->w_gate_up);
  R.wd = static_cast<const uint16_t *>(L->w_down);
  R.off = b.offsets;
  R.gates = topk_gates;
  R.perm_src = b.perm_src;
  R.perm_pos = b.perm_pos;
  R.dl = b.dl;
  if (z_saved) {   // the forward's pre-activations: no recompute
    R.z = const_cast<float *>(z_saved);
    R.z_given = 1;
  }
  R.dwgu = dw_gate_up;
  R.dwd = dw_down;
  e = moe::launch_expert_backward(R, st);
  if (e != hipSuccess) return hip_status(e, "moe_backward: routed experts");
  e = moe::launch_router_backward(b.dl, b.x_perm, b.offsets, E, H, dw_router, dbias, st);
  if (e != hipSuccess) return hip_status(e, "moe_backward: router");
  const float *dx_shared = nullptr;
  if (L->shared_inter > 0) {
    moe::BwdExpert &S = b.shared;
    S.T = T;
    S.k = 1;
    S.x = static_cast<const uint16_t *>(x);
    S.dy = static_cast<const uint16_t *>(dy);
    S.wgu = static_cast<const uint16_t *>(L->w_shared_gate_up);
    S.wd = static_cast<const uint16_t *>(L->w_shared_down);
    if (z_saved) {
      S.z = const_cast<float *>(z_saved) + (size_t)N * 2 * L->inter;
      S.z_given = 1;
    }
    S.dwgu = dw_shared_gate_up;
    S.dwd = dw_shared_down;
    e = moe::launch_expert_backward(S, st);
    if (e != hipSuccess) return hip_status(e, "moe_backward: shared expert");
    dx_shared = S.dx_rows;
  }
  e = moe::launch_dx_backward(dx_shared, R.dx_rows, b.perm_pos, topk_ids, b.dl,
                              static_cast<const uint16_t *>(L->w_router), T, k, H, dx, st);
  return hip_status(e, "moe_backward: dx");
}

moe_status moe_pack_weights(const void *src, void *dst, int64_t count, int64_t rows, int64_t row_bytes,
                            void *stream) {
  if (!src || !dst) return fail(MOE_EINVAL, "moe_pack_weights: NULL pointer");
  if (!aligned16(src) || !aligned16(dst)) return fail(MOE_EINVAL, "moe_pack_weights: pointers not 16-byte aligned");
  if (count <= 0 || rows <= 0 || rows % 16 != 0 || row_bytes <= 0 || row_bytes % 128 != 0)
    return fail(MOE_EINVAL,
                "moe_pack_weights: count %lld must be positive, rows %lld a positive multiple of 16 and row_bytes "
                "%lld of 128", (long long)count, (long long)rows, (long long)row_bytes);
  if (rows > (int64_t)1 << 40 || row_bytes > (int64_t)1 << 40 || count > ((int64_t)1 << 62) / (rows * row_bytes))
    return fail(MOE_EINVAL, "moe_pack_weights: size too large");
  const uint8_t *a = static_cast<const uint8_t *>(src);
  const uint8_t *b = static_cast<const uint8_t *>(dst);
  const int64_t n = count * rows * row_bytes;
  if (a < b + n && b < a + n) return fail(MOE_EINVAL, "moe_pack_weights: src and dst overlap");
  return hip_status(
      moe::launch_pack_tile16(a, static_cast<uint8_t *>(dst), count, rows, row_bytes, (hipStream_t)stream),
      "moe_pack_weights");
}

}  // extern "C"
