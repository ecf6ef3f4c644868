// C ABI of libgdn.so (declared in include/gdn.h): argument validation and
// dispatch to the kernel launchers.  Validation never touches the HIP runtime, so
// a call with invalid arguments returns its status and launches nothing on any
// machine.
#include "gdn.h"

#include <cmath>
#include <cstddef>
#include <cstdint>
#include <initializer_list>

#include "internal.h"

namespace {

using gdn::Geometry;

bool dtype_ok(int32_t d) { return d == GDN_DTYPE_F32 || d == GDN_DTYPE_BF16; }

gdn_status check_dims(const gdn_dims &d, int32_t act_dtype, int32_t out_dtype, Geometry *geo) {
  if (!dtype_ok(act_dtype) || !dtype_ok(out_dtype)) return GDN_ERR_INVALID_ARG;
  if (d.reserved != 0) return GDN_ERR_INVALID_ARG;
  if (d.num_k_heads < 1 || d.num_v_heads < 1 || d.head_dim_k < 1 || d.head_dim_v < 1 ||
      d.conv_kernel < 1)
    return GDN_ERR_INVALID_ARG;
  if (d.num_k_heads > 4096 || d.num_v_heads > 4096 || d.head_dim_k > 4096 || d.head_dim_v > 4096 ||
      d.conv_kernel > 64)
    return GDN_ERR_INVALID_ARG;
  if (d.num_v_heads % d.num_k_heads != 0) return GDN_ERR_INVALID_ARG;
  const int G = d.num_v_heads / d.num_k_heads;
  if (G != 1 && G != 2 && G != 4) return GDN_ERR_UNSUPPORTED;
  if (d.head_dim_k != d.head_dim_v) return GDN_ERR_UNSUPPORTED;
  if (d.head_dim_k != 32 && d.head_dim_k != 64 && d.head_dim_k != 128) return GDN_ERR_UNSUPPORTED;
  if (d.conv_kernel < 2 || d.conv_kernel > 4) return GDN_ERR_UNSUPPORTED;
  geo->Hk = d.num_k_heads;
  geo->Hv = d.num_v_heads;
  geo->D = d.head_dim_k;
  geo->K = d.conv_kernel;
  geo->conv_dim = 2 * d.num_k_heads * d.head_dim_k + d.num_v_heads * d.head_dim_v;
  geo->act_bf16 = act_dtype == GDN_DTYPE_BF16;
  geo->out_bf16 = out_dtype == GDN_DTYPE_BF16;
  return GDN_OK;
}

// Options an entry point takes: every option it does not take must be zero.
struct Opts {
  int state_f16, gates_raw, norm_sigmoid;
};
gdn_status check_opts(const gdn_options &o, bool takes_state, bool takes_gates, bool takes_norm, Opts *out) {
  if (o.reserved != 0) return GDN_ERR_INVALID_ARG;
  if (o.state_dtype != GDN_DTYPE_F32 && !(takes_state && o.state_dtype == GDN_DTYPE_F16))
    return GDN_ERR_INVALID_ARG;
  if (o.gate_mode != GDN_GATES_DIRECT && !(takes_gates && o.gate_mode == GDN_GATES_RAW))
    return GDN_ERR_INVALID_ARG;
  if (o.norm_gate != GDN_NORM_GATE_SILU && !(takes_norm && o.norm_gate == GDN_NORM_GATE_SIGMOID))
    return GDN_ERR_INVALID_ARG;
  out->state_f16 = o.state_dtype == GDN_DTYPE_F16;
  out->gates_raw = o.gate_mode == GDN_GATES_RAW;
  out->norm_sigmoid = o.norm_gate == GDN_NORM_GATE_SIGMOID;
  return GDN_OK;
}

void set_opts(gdn::RecurrentLaunch *p, const Opts &o) {
  p->state_f16 = o.state_f16;
  p->gates_raw = o.gates_raw;
  p->norm_sigmoid = o.norm_sigmoid;
}

// Floats per write-on-accept stash row: k_hat of every key head, u of every value
// head, a of every value head, rounded up to whole 16-byte vectors.
int stash_row_floats(const Geometry &g) { return (g.Hk * g.D + g.Hv * g.D + g.Hv + 3) & ~3; }

bool finite(float v) { return std::isfinite(v); }
bool eps_ok(float v) { return std::isfinite(v) && v >= 0.0f; }
// Buffers the kernels move in 8- and 16-byte vectors must start on a 16-byte boundary
// (hipMalloc and framework allocations do; a view into the middle of one may not).
bool aligned16(std::initializer_list<const void *> ps) {
  for (const void *q : ps)
    if (reinterpret_cast<uintptr_t>(q) & 15) return false;
  return true;
}

gdn_status hip_status(hipError_t e) { return e == hipSuccess ? GDN_OK : GDN_ERR_HIP; }

// Workspace layout of gdn_prefill_chunked: [front y (fp32, when x is given)]
// [o staging (fp32, when z is given)] [chunk-kernel workspace].
struct PrefillPlan {
  Geometry geo;
  bool fused_front, epilogue;
  size_t y_bytes, o_bytes, core_bytes, total;
  Opts opts;
};

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

gdn_status plan_prefill(const gdn_prefill_args *a, PrefillPlan *plan) {
  if (a == nullptr) return GDN_ERR_INVALID_ARG;
  if (a->struct_size != sizeof(gdn_prefill_args)) return GDN_ERR_INVALID_ARG;
  gdn_status s = check_dims(a->dims, a->act_dtype, a->out_dtype, &plan->geo);
  if (s != GDN_OK) return s;
  if (a->num_seqs < 0 || a->total_tokens < 0 || a->reserved != 0 || a->reserved_f != 0.0f)
    return GDN_ERR_INVALID_ARG;
  if (a->chunk_size != GDN_PREFILL_CHUNK) return GDN_ERR_UNSUPPORTED;
  if (a->total_tokens > ((int64_t)1 << 31) - 1) return GDN_ERR_INVALID_ARG;
  if (a->total_tokens > 0 && a->num_seqs == 0) return GDN_ERR_INVALID_ARG;
  if (!finite(a->scale) || !eps_ok(a->l2_eps) || !eps_ok(a->norm_eps)) return GDN_ERR_INVALID_ARG;
  s = check_opts(a->opt, true, true, true, &plan->opts);
  if (s != GDN_OK) return s;
  plan->fused_front = a->x != nullptr;
  plan->epilogue = a->z != nullptr;
  const int64_t T = a->total_tokens;
  const Geometry &g = plan->geo;
  plan->y_bytes = plan->fused_front ? align256((size_t)T * g.conv_dim * 4) : 0;
  plan->o_bytes = plan->epilogue ? align256((size_t)T * g.Hv * g.D * 4) : 0;
  // y: fp32 from the fused front, else the caller's rows in the activation dtype
  const bool y_bf16 = !plan->fused_front && g.act_bf16;
  plan->core_bytes = a->num_seqs > 0 ? align256(gdn::prefill_core_workspace(g, a->num_seqs, T, y_bf16)) : 0;
  plan->total = plan->y_bytes + plan->o_bytes + plan->core_bytes;
  return GDN_OK;
}

}  // namespace

extern "C" {

const char *gdn_status_string(gdn_status status) {
  switch (status) {
    case GDN_OK: return "GDN_OK";
    case GDN_ERR_INVALID_ARG: return "GDN_ERR_INVALID_ARG: invalid argument";
    case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED: no kernel for this shape";
    case GDN_ERR_WORKSPACE: return "GDN_ERR_WORKSPACE: workspace missing or too small";
    case GDN_ERR_HIP: return "GDN_ERR_HIP: the HIP runtime reported an error";
  }
  return "unknown gdn_status";
}

int32_t gdn_abi_version(void) { return GDN_ABI_VERSION; }

gdn_status gdn_conv_l2norm(const gdn_conv_args *a, void *stream) {
  if (a == nullptr || a->struct_size != sizeof(gdn_conv_args)) return GDN_ERR_INVALID_ARG;
  gdn::ConvLaunch p{};
  gdn_status s = check_dims(a->dims, a->act_dtype, a->out_dtype, &p.geo);
  if (s != GDN_OK) return s;
  if (a->num_seqs < 0 || a->total_tokens < 0 || !eps_ok(a->l2_eps)) return GDN_ERR_INVALID_ARG;
  if (a->total_tokens > ((int64_t)1 << 31) - 1) return GDN_ERR_INVALID_ARG;
  if (a->total_tokens > 0 && a->num_seqs == 0) return GDN_ERR_INVALID_ARG;
  if (a->num_seqs > 0 && (a->cu_seqlens == nullptr || a->conv_w == nullptr || a->conv_state == nullptr))
    return GDN_ERR_INVALID_ARG;
  if (a->total_tokens > 0 && (a->x == nullptr || a->y == nullptr)) return GDN_ERR_INVALID_ARG;
  if (a->x != nullptr && a->x == a->y) return GDN_ERR_INVALID_ARG;
  if (!aligned16({a->x, a->y, a->conv_w})) return GDN_ERR_INVALID_ARG;
  if (a->num_seqs > 65535) return GDN_ERR_INVALID_ARG;
  p.n = a->num_seqs;
  p.T = a->total_tokens;
  p.cu = a->cu_seqlens;
  p.x = a->x;
  p.conv_w = a->conv_w;
  p.conv_state = a->conv_state;
  p.y = a->y;
  p.y_f32 = 0;
  p.l2_eps = a->l2_eps;
  return hip_status(gdn::launch_conv_l2norm(p, static_cast<hipStream_t>(stream)));
}

gdn_status gdn_decode_batched(const gdn_decode_args *a, void *stream) {
  if (a == nullptr || a->struct_size != sizeof(gdn_decode_args)) return GDN_ERR_INVALID_ARG;
  gdn::RecurrentLaunch p{};
  gdn_status s = check_dims(a->dims, a->act_dtype, a->out_dtype, &p.geo);
  if (s != GDN_OK) return s;
  if (a->num_seqs < 0 || a->reserved_f != 0.0f) return GDN_ERR_INVALID_ARG;
  if (!finite(a->scale) || !eps_ok(a->l2_eps) || !eps_ok(a->norm_eps)) return GDN_ERR_INVALID_ARG;
  if ((int64_t)a->num_seqs * p.geo.Hk > ((int64_t)1 << 31) - 1) return GDN_ERR_INVALID_ARG;
  if (a->num_seqs > 0 &&
      (a->x == nullptr || a->conv_w == nullptr || a->conv_state == nullptr || a->a == nullptr ||
       a->b == nullptr || a->h_state == nullptr || a->out == nullptr))
    return GDN_ERR_INVALID_ARG;
  if (a->z != nullptr && a->norm_w == nullptr) return GDN_ERR_INVALID_ARG;
  if (!aligned16({a->x, a->conv_w, a->z, a->norm_w, a->out})) return GDN_ERR_INVALID_ARG;
  Opts o;
  s = check_opts(a->opt, true, true, true, &o);
  if (s != GDN_OK) return s;
  set_opts(&p, o);
  p.n = a->num_seqs;
  p.mode = gdn::kModeDecode;
  p.cu = nullptr;
  p.x = a->x;
  p.conv_w = a->conv_w;
  p.conv_state = a->conv_state;
  p.a = a->a;
  p.b = a->b;
  p.states = a->h_state;
  p.z = a->z;
  p.norm_w = a->norm_w;
  p.out = a->out;
  p.scale = a->scale;
  p.l2_eps = a->l2_eps;
  p.norm_eps = a->norm_eps;
  return hip_status(gdn::launch_recurrent(p, static_cast<hipStream_t>(stream)));
}

gdn_status gdn_verify_multi(const gdn_verify_args *a, void *stream) {
  if (a == nullptr || a->struct_size != sizeof(gdn_verify_args)) return GDN_ERR_INVALID_ARG;
  gdn::RecurrentLaunch p{};
  gdn_status s = check_dims(a->dims, a->act_dtype, a->out_dtype, &p.geo);
  if (s != GDN_OK) return s;
  if (a->num_seqs < 0 || a->num_seqs > GDN_VERIFY_WY_TABLE_SEQS) return GDN_ERR_INVALID_ARG;
  if (a->max_k < GDN_VERIFY_MIN_K || a->max_k > GDN_VERIFY_MAX_K) return GDN_ERR_INVALID_ARG;
  if (a->total_rows < 0 || a->total_rows > a->num_seqs * a->max_k) return GDN_ERR_INVALID_ARG;
  if (a->reserved != 0 || a->reserved_f != 0.0f) return GDN_ERR_INVALID_ARG;
  if (!finite(a->scale) || !eps_ok(a->l2_eps) || !eps_ok(a->norm_eps)) return GDN_ERR_INVALID_ARG;
  if (a->num_seqs > 0 &&
      (a->cu_ks == nullptr || a->x == nullptr || a->conv_w == nullptr || a->conv_state == nullptr ||
       a->a == nullptr || a->b == nullptr || a->wy_tables == nullptr || a->out == nullptr))
    return GDN_ERR_INVALID_ARG;
  if (a->z != nullptr && a->norm_w == nullptr) return GDN_ERR_INVALID_ARG;
  if (!aligned16({a->x, a->conv_w, a->z, a->norm_w, a->out})) return GDN_ERR_INVALID_ARG;
  Opts o;
  s = check_opts(a->opt, true, true, true, &o);
  if (s != GDN_OK) return s;
  set_opts(&p, o);
  p.n = a->num_seqs;
  p.mode = gdn::kModeVerify;
  p.cu = a->cu_ks;
  p.x = a->x;
  p.conv_w = a->conv_w;
  p.conv_state = a->conv_state;
  p.a = a->a;
  p.b = a->b;
  p.states = a->wy_tables;
  p.z = a->z;
  p.norm_w = a->norm_w;
  p.out = a->out;
  p.scale = a->scale;
  p.l2_eps = a->l2_eps;
  p.norm_eps = a->norm_eps;
  return hip_status(gdn::launch_recurrent(p, static_cast<hipStream_t>(stream)));
}

gdn_status gdn_verify_commit(const gdn_commit_args *a, void *stream) {
  if (a == nullptr || a->struct_size != sizeof(gdn_commit_args)) return GDN_ERR_INVALID_ARG;
  gdn::CommitLaunch p{};
  gdn_status s = check_dims(a->dims, a->act_dtype, GDN_DTYPE_F32, &p.geo);
  if (s != GDN_OK) return s;
  if (a->num_seqs < 0 || a->num_seqs > GDN_VERIFY_WY_TABLE_SEQS || a->reserved != 0)
    return GDN_ERR_INVALID_ARG;
  if (a->num_seqs > 0 && (a->cu_ks == nullptr || a->n_accepted == nullptr || a->wy_tables == nullptr ||
                          a->x == nullptr || a->conv_state == nullptr))
    return GDN_ERR_INVALID_ARG;
  if (!aligned16({a->x})) return GDN_ERR_INVALID_ARG;
  Opts o;
  s = check_opts(a->opt, true, false, false, &o);
  if (s != GDN_OK) return s;
  p.state_f16 = o.state_f16;
  p.n = a->num_seqs;
  p.cu = a->cu_ks;
  p.n_accepted = a->n_accepted;
  p.tables = a->wy_tables;
  p.x = a->x;
  p.conv_state = a->conv_state;
  return hip_status(gdn::launch_commit(p, static_cast<hipStream_t>(stream)));
}

gdn_status gdn_gated_rmsnorm(const gdn_norm_args *a, void *stream) {
  if (a == nullptr || a->struct_size != sizeof(gdn_norm_args)) return GDN_ERR_INVALID_ARG;
  if (!dtype_ok(a->in_dtype) || !dtype_ok(a->act_dtype) || !dtype_ok(a->out_dtype))
    return GDN_ERR_INVALID_ARG;
  const gdn_dims &d = a->dims;
  if (d.num_v_heads < 1 || d.num_v_heads > 4096 || d.head_dim_v < 1 || a->total_tokens < 0 ||
      a->reserved_f != 0.0f || !eps_ok(a->eps))
    return GDN_ERR_INVALID_ARG;
  if (d.head_dim_v != 32 && d.head_dim_v != 64 && d.head_dim_v != 128) return GDN_ERR_UNSUPPORTED;
  if (a->total_tokens * d.num_v_heads > ((int64_t)1 << 33)) return GDN_ERR_INVALID_ARG;
  if (a->total_tokens > 0 && (a->o == nullptr || a->z == nullptr || a->norm_w == nullptr || a->out == nullptr))
    return GDN_ERR_INVALID_ARG;
  if (!aligned16({a->o, a->z, a->norm_w, a->out})) return GDN_ERR_INVALID_ARG;
  Opts o;
  gdn_status s = check_opts(a->opt, false, false, true, &o);
  if (s != GDN_OK) return s;
  gdn::NormLaunch p{};
  p.norm_sigmoid = o.norm_sigmoid;
  p.Hv = d.num_v_heads;
  p.D = d.head_dim_v;
  p.T = a->total_tokens;
  p.in_bf16 = a->in_dtype == GDN_DTYPE_BF16;
  p.act_bf16 = a->act_dtype == GDN_DTYPE_BF16;
  p.out_bf16 = a->out_dtype == GDN_DTYPE_BF16;
  p.o = a->o;
  p.z = a->z;
  p.norm_w = a->norm_w;
  p.out = a->out;
  p.eps = a->eps;
  return hip_status(gdn::launch_gated_rmsnorm(p, static_cast<hipStream_t>(stream)));
}

gdn_status gdn_prefill_workspace_bytes(const gdn_prefill_args *a, size_t *bytes) {
  if (bytes == nullptr) return GDN_ERR_INVALID_ARG;
  *bytes = 0;
  PrefillPlan plan;
  gdn_status s = plan_prefill(a, &plan);
  if (s != GDN_OK) return s;
  *bytes = plan.total;
  return GDN_OK;
}

}  // extern "C"

namespace {

// Validation shared by both prefill entry points (everything but the workspace).
gdn_status check_prefill(const gdn_prefill_args *a, PrefillPlan *plan) {
  gdn_status s = plan_prefill(a, plan);
  if (s != GDN_OK) return s;
  const int n = a->num_seqs;
  const int64_t T = a->total_tokens;
  if (n > 0 && (a->cu_seqlens == nullptr || a->h_state == nullptr)) return GDN_ERR_INVALID_ARG;
  // per-token arrays are read only when there are tokens
  if (T > 0 && (a->a == nullptr || a->b == nullptr)) return GDN_ERR_INVALID_ARG;
  if (T > 0 && a->out == nullptr) return GDN_ERR_INVALID_ARG;
  if (plan->fused_front && (a->conv_w == nullptr || a->conv_state == nullptr)) return GDN_ERR_INVALID_ARG;
  if (!plan->fused_front && T > 0 && a->y == nullptr) return GDN_ERR_INVALID_ARG;
  if (plan->epilogue && a->norm_w == nullptr) return GDN_ERR_INVALID_ARG;
  if (n > 65535) return GDN_ERR_INVALID_ARG;
  if (!aligned16({a->y, a->x, a->conv_w, a->z, a->norm_w, a->out, a->workspace})) return GDN_ERR_INVALID_ARG;
  return GDN_OK;
}

// The launches of a validated prefill on the workspace ws (plan.total bytes).
gdn_status run_prefill(const gdn_prefill_args *a, const PrefillPlan &plan, char *ws, hipStream_t st) {
  const int n = a->num_seqs;
  const int64_t T = a->total_tokens;
  const Geometry &g = plan.geo;

  const void *y = a->y;
  int y_bf16 = g.act_bf16;
  if (plan.fused_front) {
    gdn::ConvLaunch c{};
    c.geo = g;
    c.n = n;
    c.T = T;
    c.cu = a->cu_seqlens;
    c.x = a->x;
    c.conv_w = a->conv_w;
    c.conv_state = a->conv_state;
    c.y = ws;
    c.y_f32 = 1;
    c.l2_eps = a->l2_eps;
    hipError_t e = gdn::launch_conv_l2norm(c, st);
    if (e != hipSuccess) return GDN_ERR_HIP;
    y = ws;
    y_bf16 = 0;
  }
  gdn::PrefillLaunch p{};
  p.geo = g;
  p.n = n;
  p.T = T;
  p.cu = a->cu_seqlens;
  p.y = y;
  p.y_bf16 = y_bf16;
  p.a = a->a;
  p.b = a->b;
  p.gates_raw = plan.opts.gates_raw;
  p.h_state = a->h_state;
  p.state_f16 = plan.opts.state_f16;
  p.o = plan.epilogue ? static_cast<void *>(ws + plan.y_bytes) : a->out;
  p.o_f32 = plan.epilogue ? 1 : 0;
  p.scale = a->scale;
  p.workspace = ws + plan.y_bytes + plan.o_bytes;
  hipError_t e = gdn::launch_prefill(p, st);
  if (e != hipSuccess) return GDN_ERR_HIP;
  if (plan.epilogue && T > 0) {
    gdn::NormLaunch nl{};
    nl.Hv = g.Hv;
    nl.D = g.D;
    nl.T = T;
    nl.in_bf16 = 0;
    nl.act_bf16 = g.act_bf16;
    nl.out_bf16 = g.out_bf16;
    nl.norm_sigmoid = plan.opts.norm_sigmoid;
    nl.o = p.o;
    nl.z = a->z;
    nl.norm_w = a->norm_w;
    nl.out = a->out;
    nl.eps = a->norm_eps;
    e = gdn::launch_gated_rmsnorm(nl, st);
    if (e != hipSuccess) return GDN_ERR_HIP;
  }
  return GDN_OK;
}

static_assert(gdn::kPrefillScratchBytes == GDN_PREFILL_SCRATCH_BYTES, "scratch size of the header");

}  // namespace

extern "C" {

gdn_status gdn_prefill_chunked(const gdn_prefill_args *a, void *stream) {
  PrefillPlan plan;
  gdn_status s = check_prefill(a, &plan);
  if (s != GDN_OK) return s;
  if (plan.total > 0 && (a->workspace == nullptr || a->workspace_bytes < plan.total))
    return GDN_ERR_WORKSPACE;
  if (a->num_seqs == 0) return GDN_OK;
  return run_prefill(a, plan, static_cast<char *>(a->workspace), static_cast<hipStream_t>(stream));
}

gdn_status gdn_prefill_chunked_noalloc(const gdn_prefill_args *a, void *stream) {
  PrefillPlan plan;
  gdn_status s = check_prefill(a, &plan);
  if (s != GDN_OK) return s;
  if (a->workspace != nullptr || a->workspace_bytes != 0) return GDN_ERR_INVALID_ARG;
  if (plan.total > gdn::kPrefillScratchBytes) return GDN_ERR_WORKSPACE;
  if (a->num_seqs == 0) return GDN_OK;
  void *ws = nullptr;
  if (gdn::prefill_scratch(&ws) != hipSuccess) return GDN_ERR_HIP;
  return run_prefill(a, plan, static_cast<char *>(ws), static_cast<hipStream_t>(stream));
}

gdn_status gdn_woa_stash_bytes(const gdn_woa_args *a, size_t *bytes) {
  if (bytes == nullptr) return GDN_ERR_INVALID_ARG;
  *bytes = 0;
  if (a == nullptr || a->struct_size != sizeof(gdn_woa_args)) return GDN_ERR_INVALID_ARG;
  Geometry geo;
  gdn_status s = check_dims(a->dims, a->act_dtype, a->out_dtype, &geo);
  if (s != GDN_OK) return s;
  if (a->total_rows < 0) return GDN_ERR_INVALID_ARG;
  *bytes = (size_t)a->total_rows * stash_row_floats(geo) * sizeof(float);
  return GDN_OK;
}

gdn_status gdn_verify_woa(const gdn_woa_args *a, void *stream) {
  if (a == nullptr || a->struct_size != sizeof(gdn_woa_args)) return GDN_ERR_INVALID_ARG;
  gdn::RecurrentLaunch p{};
  gdn_status s = check_dims(a->dims, a->act_dtype, a->out_dtype, &p.geo);
  if (s != GDN_OK) return s;
  if (a->num_seqs < 0 || a->num_seqs > GDN_VERIFY_WY_TABLE_SEQS) return GDN_ERR_INVALID_ARG;
  if (a->max_k < GDN_VERIFY_MIN_K || a->max_k > GDN_VERIFY_MAX_K) return GDN_ERR_INVALID_ARG;
  if (a->total_rows < 0 || a->total_rows > a->num_seqs * a->max_k) return GDN_ERR_INVALID_ARG;
  if (a->reserved != 0 || a->reserved_f != 0.0f) return GDN_ERR_INVALID_ARG;
  if (!finite(a->scale) || !eps_ok(a->l2_eps) || !eps_ok(a->norm_eps)) return GDN_ERR_INVALID_ARG;
  if (a->num_seqs > 0 &&
      (a->cu_ks == nullptr || a->x == nullptr || a->conv_w == nullptr || a->conv_state == nullptr ||
       a->a == nullptr || a->b == nullptr || a->h_state == nullptr || a->out == nullptr))
    return GDN_ERR_INVALID_ARG;
  if (a->z != nullptr && a->norm_w == nullptr) return GDN_ERR_INVALID_ARG;
  if (!aligned16({a->x, a->conv_w, a->z, a->norm_w, a->out, a->stash})) return GDN_ERR_INVALID_ARG;
  Opts o;
  s = check_opts(a->opt, true, true, true, &o);
  if (s != GDN_OK) return s;
  const size_t need = (size_t)a->total_rows * stash_row_floats(p.geo) * sizeof(float);
  if (a->num_seqs > 0 && (a->stash == nullptr || a->stash_bytes < need)) return GDN_ERR_WORKSPACE;
  set_opts(&p, o);
  p.n = a->num_seqs;
  p.mode = gdn::kModeWoa;
  p.cu = a->cu_ks;
  p.x = a->x;
  p.conv_w = a->conv_w;
  p.conv_state = a->conv_state;
  p.a = a->a;
  p.b = a->b;
  p.states = a->h_state;
  p.z = a->z;
  p.norm_w = a->norm_w;
  p.out = a->out;
  p.stash = a->stash;
  p.stash_row = stash_row_floats(p.geo);
  p.scale = a->scale;
  p.l2_eps = a->l2_eps;
  p.norm_eps = a->norm_eps;
  return hip_status(gdn::launch_recurrent(p, static_cast<hipStream_t>(stream)));
}

gdn_status gdn_fold_accepted(const gdn_fold_args *a, void *stream) {
  if (a == nullptr || a->struct_size != sizeof(gdn_fold_args)) return GDN_ERR_INVALID_ARG;
  gdn::FoldLaunch p{};
  gdn_status s = check_dims(a->dims, a->act_dtype, GDN_DTYPE_F32, &p.geo);
  if (s != GDN_OK) return s;
  if (a->num_seqs < 0 || a->num_seqs > GDN_VERIFY_WY_TABLE_SEQS || a->total_rows < 0) return GDN_ERR_INVALID_ARG;
  if (a->num_seqs > 0 && (a->cu_ks == nullptr || a->n_accepted == nullptr || a->h_state == nullptr ||
                          a->x == nullptr || a->conv_state == nullptr))
    return GDN_ERR_INVALID_ARG;
  if (!aligned16({a->x, a->stash})) return GDN_ERR_INVALID_ARG;
  Opts o;
  s = check_opts(a->opt, true, false, false, &o);
  if (s != GDN_OK) return s;
  const size_t need = (size_t)a->total_rows * stash_row_floats(p.geo) * sizeof(float);
  if (a->num_seqs > 0 && (a->stash == nullptr || a->stash_bytes < need)) return GDN_ERR_WORKSPACE;
  p.n = a->num_seqs;
  p.state_f16 = o.state_f16;
  p.cu = a->cu_ks;
  p.n_accepted = a->n_accepted;
  p.states = a->h_state;
  p.stash = a->stash;
  p.stash_row = stash_row_floats(p.geo);
  p.x = a->x;
  p.conv_state = a->conv_state;
  return hip_status(gdn::launch_fold(p, static_cast<hipStream_t>(stream)));
}

gdn_status gdn_decode_tokens(const gdn_tokens_args *a, void *stream) {
  if (a == nullptr || a->struct_size != sizeof(gdn_tokens_args)) return GDN_ERR_INVALID_ARG;
  gdn::RecurrentLaunch p{};
  gdn_status s = check_dims(a->dims, a->act_dtype, a->out_dtype, &p.geo);
  if (s != GDN_OK) return s;
  if (a->num_seqs < 0 || a->num_seqs > GDN_VERIFY_WY_TABLE_SEQS) return GDN_ERR_INVALID_ARG;
  if (a->max_tokens < 1 || a->max_tokens > GDN_DECODE_MAX_TOKENS) return GDN_ERR_INVALID_ARG;
  if (a->total_rows < 0 || a->total_rows > a->num_seqs * a->max_tokens) return GDN_ERR_INVALID_ARG;
  if (a->reserved != 0 || a->reserved_f != 0.0f) return GDN_ERR_INVALID_ARG;
  if (!finite(a->scale) || !eps_ok(a->l2_eps) || !eps_ok(a->norm_eps)) return GDN_ERR_INVALID_ARG;
  if (a->num_seqs > 0 &&
      (a->cu_tokens == nullptr || a->x == nullptr || a->conv_w == nullptr || a->conv_state == nullptr ||
       a->a == nullptr || a->b == nullptr || a->h_state == nullptr || a->out == nullptr))
    return GDN_ERR_INVALID_ARG;
  if (a->z != nullptr && a->norm_w == nullptr) return GDN_ERR_INVALID_ARG;
  if (!aligned16({a->x, a->conv_w, a->z, a->norm_w, a->out})) return GDN_ERR_INVALID_ARG;
  Opts o;
  s = check_opts(a->opt, true, true, true, &o);
  if (s != GDN_OK) return s;
  set_opts(&p, o);
  p.n = a->num_seqs;
  p.mode = gdn::kModeTokens;
  p.cu = a->cu_tokens;
  p.x = a->x;
  p.conv_w = a->conv_w;
  p.conv_state = a->conv_state;
  p.a = a->a;
  p.b = a->b;
  p.states = a->h_state;
  p.z = a->z;
  p.norm_w = a->norm_w;
  p.out = a->out;
  p.scale = a->scale;
  p.l2_eps = a->l2_eps;
  p.norm_eps = a->norm_eps;
  return hip_status(gdn::launch_recurrent(p, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
