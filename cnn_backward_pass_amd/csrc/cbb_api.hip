// cbb_api.hip -- the extern "C" entry points of libcbb.so: argument checks on
// the host (before any HIP call), workspace carving, and kernel enqueue on the
// caller's stream.  See include/cbb.h for the contract of every call.
#include <cstdio>
#include <cstring>

#include "cbb_internal.h"

using namespace cbb;

namespace {

constexpr int64_t kMaxIndex = (int64_t)1 << 31;  // per-tensor element counts must index in int32
constexpr size_t kAlign = 256;

inline hipStream_t S(void* s) { return reinterpret_cast<hipStream_t>(s); }

struct ConvPlan {
  int64_t oh, ow;
  size_t part_bytes, dw_bytes, below_bytes, total;
};

int check_desc(const cbb_conv_desc* d, ConvPlan* plan) {
  if (!d) return CBB_EINVAL;
  if (d->batch < 1 || d->in_c < 1 || d->in_h < 1 || d->in_w < 1 || d->out_c < 1 ||
      d->ksize < 1 || d->stride < 1 || d->pad < 0)
    return CBB_EINVAL;
  if (d->act < CBB_ACT_LINEAR || d->act > CBB_ACT_LOGGY) return CBB_EINVAL;
  if (d->batch_normalize < CBB_BN_NONE || d->batch_normalize > CBB_BN_FIXED) return CBB_EINVAL;
  if (d->batch_normalize && !(d->bn_eps > 0.f)) return CBB_EINVAL;
  if (d->groups < 0 || d->dilation < 0) return CBB_EINVAL;
  const int groups = d->groups > 1 ? d->groups : 1, dil = d->dilation > 1 ? d->dilation : 1;
  if (d->in_c % groups || d->out_c % groups) return CBB_EINVAL;
  if (d->ksize > 7 || d->stride > 4 || dil > 16 || d->pad > dil * (d->ksize - 1))
    return CBB_EUNSUPPORTED;
  const int64_t span = (int64_t)dil * (d->ksize - 1) + 1;   // input pixels under one window
  const int64_t oh = ((int64_t)d->in_h + 2 * d->pad - span) / d->stride + 1;
  const int64_t ow = ((int64_t)d->in_w + 2 * d->pad - span) / d->stride + 1;
  if ((int64_t)d->in_h + 2 * d->pad < span || (int64_t)d->in_w + 2 * d->pad < span || oh < 1 ||
      ow < 1)
    return CBB_ESHAPE;
  const int64_t nx = (int64_t)d->batch * d->in_c * d->in_h * d->in_w;
  const int64_t ny = (int64_t)d->batch * d->out_c * oh * ow;
  const int64_t nw = (int64_t)d->out_c * (d->in_c / groups) * d->ksize * d->ksize;
  if (nx >= kMaxIndex || ny >= kMaxIndex || nw >= kMaxIndex) return CBB_EUNSUPPORTED;
  if (plan) {
    plan->oh = oh;
    plan->ow = ow;
    const ConvGeom g = make_geom(*d);
    // act/BN partials, then the per-channel map of a block whose dz is formed by
    // the gradient kernel (3 floats per channel)
    plan->part_bytes = align_up(actbn_workspace(d->batch, d->out_c, oh * ow), kAlign) +
                       align_up((size_t)3 * d->out_c * sizeof(float), kAlign);
    // dW and dX run one after the other on the stream (or as one fused kernel)
    // and share the second region
    plan->dw_bytes = align_up(
        std::max({conv_dw_workspace(g), conv_dx_workspace(g), conv_fused_workspace(g)}), kAlign);
    // partials of the act/BN sums of the block below (cbb_conv_block_backward_ex):
    // those of the stride-2 input-gradient kernel, or of a reduction pass over dx
    plan->below_bytes = align_up(
        std::max(bn_sums_workspace(d->batch, d->in_c, (int64_t)d->in_h * d->in_w),
                 (size_t)kDxS2pGroups * d->in_c * sizeof(float2)),
        kAlign);
    plan->total = plan->part_bytes + plan->dw_bytes + plan->below_bytes;
  }
  return CBB_OK;
}

// The rules of cbb_block_opts (see include/cbb.h).
int check_block_opts(const cbb_conv_desc* d, const float* dx, const cbb_block_opts* o) {
  if (!o) return CBB_OK;
  if (o->sums && d->batch_normalize != CBB_BN_BATCH) return CBB_EINVAL;
  if (o->below_apply_act != 0 && o->below_apply_act != 1) return CBB_EINVAL;
  if (o->below_apply_act && !o->below_sums) return CBB_EINVAL;
  if (o->below_sums) {
    if (!dx || !o->below_x_norm) return CBB_EINVAL;
    if (o->below_act < CBB_ACT_LINEAR || o->below_act > CBB_ACT_LOGGY) return CBB_EINVAL;
    if (o->below_act != CBB_ACT_LINEAR && !o->below_y) return CBB_EINVAL;
    if (o->below_sums == o->sums) return CBB_EINVAL;
  } else if (o->below_y || o->below_x_norm) {
    return CBB_EINVAL;   // the block below's tensors without a place for its sums
  }
  return CBB_OK;
}

// The block below's act/BN sums into opts->below_sums: folded from the partials
// the input-gradient kernel wrote (bb->nseg > 0; that kernel also stored g when
// asked), else a reduction pass over dx, then (below_apply_act) dx *= act'(y).
int below_sums(const cbb_conv_desc* d, float* dx, const cbb_block_opts* o, const BnBelow* bb,
               char* ws, hipStream_t st) {
  float2* out = reinterpret_cast<float2*>(o->below_sums);
  if (bb && bb->nseg > 0) return launch_bn_sums_fold(bb->part, d->in_c, bb->nseg, out, st);
  const bool lin = o->below_act == CBB_ACT_LINEAR;
  const int64_t hw = (int64_t)d->in_h * d->in_w;
  int rc = launch_bn_sums(d->batch, d->in_c, hw, dx, lin ? nullptr : o->below_y, o->below_x_norm,
                          o->below_act, o->below_slope, ws, out, st);
  if (rc || !o->below_apply_act || lin) return rc;
  return launch_act_backward(o->below_act, o->below_slope, o->below_y, dx, dx,
                             (int64_t)d->batch * d->in_c * hw, st);
}

// dW and (when dx is given) dX from dz: one fused kernel for the layers it
// covers, else the two gradient kernels one after the other.
int launch_weights_data(const ConvGeom& g, const float* x, const float* w, const float* dz,
                        float* dw, float* dx, int dx_accumulate, float* ws, hipStream_t st) {
  const bool aligned = ((uintptr_t)x % 16 == 0) && ((uintptr_t)dz % 16 == 0);
  if (dx && aligned && conv_fused_dwdx_ok(g))
    return launch_conv_fused_dwdx(g, x, w, dz, dw, dx, dx_accumulate, ws, st);
  int rc = launch_conv_dw(g, x, dz, dw, ws, st);
  if (rc || !dx) return rc;
  return launch_conv_dx(g, w, dz, dx, dx_accumulate, ws, st);
}

}  // namespace

extern "C" {

int cbb_abi_version(void) { return CBB_ABI_VERSION; }

const char* cbb_last_error(void) { return last_error_text(); }

const char* cbb_status_string(int status) {
  switch (status) {
    case CBB_OK: return "ok";
    case CBB_EINVAL: return "invalid argument (NULL pointer, non-positive size or bad enum)";
    case CBB_ESHAPE: return "inconsistent or empty shape";
    case CBB_EUNSUPPORTED: return "unsupported configuration";
    case CBB_EWORKSPACE: return "workspace missing or too small";
    case CBB_EHIP: return last_error_text()[0] ? last_error_text() : "HIP error";
    case CBB_ESCRATCH:
      return "the call needs more scratch than the static buffer of "
             "cbb_conv_block_backward_noalloc holds (CBB_NOALLOC_SCRATCH_BYTES)";
  }
  return "unknown status";
}

int cbb_conv_block_workspace_size(const cbb_conv_desc* desc, size_t* bytes) {
  if (!bytes) return CBB_EINVAL;
  ConvPlan p;
  const int rc = check_desc(desc, &p);
  if (rc) return rc;
  *bytes = p.total;
  return CBB_OK;
}

}  // extern "C"

namespace cbb {

// The argument rules of cbb_conv_block_backward other than the workspace's.
int check_block_backward(const cbb_conv_desc* desc, const float* x, const float* w,
                         const float* y, const float* x_norm, const float* var,
                         const float* gamma, const float* delta, const float* dz,
                         const float* dw, const float* db, const float* dgamma, const float* dx,
                         int dx_accumulate) {
  const int rc = check_desc(desc, nullptr);
  if (rc) return rc;
  const int bn = desc->batch_normalize, act = desc->act;
  if (!x || !w || !delta || !dw || !db) return CBB_EINVAL;
  if (act != CBB_ACT_LINEAR && !y) return CBB_EINVAL;
  if (bn && (!x_norm || !var || !gamma || !dgamma)) return CBB_EINVAL;
  if (!bn && (x_norm || var || gamma || dgamma)) return CBB_EINVAL;
  const bool passthrough = act == CBB_ACT_LINEAR && !bn;  // dz is delta itself
  // dz = NULL: not stored; the fused dW + dX kernel forms it as it stages delta
  if (!passthrough && !dz) {
    auto a16 = [](const void* q) { return !q || (uintptr_t)q % 16 == 0; };
    if (!dx || !conv_fused_dwdx_ok(make_geom(*desc)) || !a16(x) || !a16(delta) || !a16(y) ||
        !a16(x_norm))
      return CBB_EINVAL;
  }
  if (dx_accumulate != 0 && dx_accumulate != 1) return CBB_EINVAL;
  return CBB_OK;
}

}  // namespace cbb

extern "C" {

int cbb_conv_block_backward(const cbb_conv_desc* desc, const float* x, const float* w,
                            const float* y, const float* x_norm, const float* var,
                            const float* gamma, const float* delta, float* dz, float* dw,
                            float* db, float* dgamma, float* dx, int dx_accumulate,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return cbb_conv_block_backward_ex(desc, x, w, y, x_norm, var, gamma, delta, dz, dw, db, dgamma,
                                    dx, dx_accumulate, nullptr, workspace, workspace_bytes,
                                    stream);
}

int cbb_conv_block_backward_ex(const cbb_conv_desc* desc, const float* x, const float* w,
                               const float* y, const float* x_norm, const float* var,
                               const float* gamma, const float* delta, float* dz, float* dw,
                               float* db, float* dgamma, float* dx, int dx_accumulate,
                               const cbb_block_opts* opts, void* workspace,
                               size_t workspace_bytes, void* stream) {
  ConvPlan p;
  int rc = check_block_backward(desc, x, w, y, x_norm, var, gamma, delta, dz, dw, db, dgamma, dx,
                                dx_accumulate);
  if (rc) return rc;
  rc = check_block_opts(desc, dx, opts);
  if (rc) return rc;
  check_desc(desc, &p);
  const float2* sums_in = opts ? reinterpret_cast<const float2*>(opts->sums) : nullptr;
  const bool below = opts && opts->below_sums;
  const int bn = desc->batch_normalize, act = desc->act;
  const bool passthrough = act == CBB_ACT_LINEAR && !bn;  // dz is delta itself
  const ConvGeom g = make_geom(*desc);
  const bool form_dz = !passthrough && !dz;
  if (p.total > 0 && (!workspace || workspace_bytes < p.total)) return CBB_EWORKSPACE;
  if (workspace && ((uintptr_t)workspace % kAlign)) return CBB_EWORKSPACE;

  hipStream_t st = S(stream);
  char* ws = static_cast<char*>(workspace);
  if (form_dz) {
    float* coef = reinterpret_cast<float*>(
        ws + align_up(actbn_workspace(desc->batch, desc->out_c, p.oh * p.ow), kAlign));
    rc = launch_actbn(desc->batch, desc->out_c, p.oh * p.ow, delta, y, x_norm, act, desc->slope,
                      var, gamma, desc->bn_eps, bn, nullptr, dgamma, db, ws, st, coef, sums_in);
    if (rc) return rc;
    const DzSource src{act == CBB_ACT_LINEAR ? nullptr : y,
                       bn == CBB_BN_BATCH ? x_norm : nullptr, coef, act, desc->slope};
    rc = launch_conv_fused_dwdx(g, x, w, delta, dw, dx, dx_accumulate,
                                reinterpret_cast<float*>(ws + p.part_bytes), st, &src);
    if (rc || !below) return rc;
    return below_sums(desc, dx, opts, nullptr, ws + p.part_bytes + p.dw_bytes, st);
  }
  // Batch statistics with dz stored: on the layers the 3x3 row-streaming dW kernel
  // takes, that kernel forms dz from delta, y and x_norm and writes it for the
  // input gradient, so the act/BN stage stops after the sums (no apply pass).
  auto a16 = [](const void* q) { return !q || (uintptr_t)q % 16 == 0; };
  if (bn == CBB_BN_BATCH && dz && dz != delta && dz != y && dz != x_norm &&
      conv_dw_forms_dz_ok(g) && a16(x) && a16(delta) && a16(y) && a16(x_norm) && a16(dz)) {
    float* coef = reinterpret_cast<float*>(
        ws + align_up(actbn_workspace(desc->batch, desc->out_c, p.oh * p.ow), kAlign));
    rc = launch_actbn(desc->batch, desc->out_c, p.oh * p.ow, delta, y, x_norm, act, desc->slope,
                      var, gamma, desc->bn_eps, bn, nullptr, dgamma, db, ws, st, coef, sums_in);
    if (rc) return rc;
    const DzSource src{act == CBB_ACT_LINEAR ? nullptr : y, x_norm, coef, act, desc->slope};
    float* ws2 = reinterpret_cast<float*>(ws + p.part_bytes);
    rc = launch_conv_dw_forming_dz(g, x, delta, src, dz, dw, ws2, st);
    if (rc || !dx) return rc;
    char* wsb = ws + p.part_bytes + p.dw_bytes;
    BnBelow bb{opts && below ? opts->below_y : nullptr, below ? opts->below_x_norm : nullptr,
               below ? opts->below_act : 0, below ? opts->below_slope : 0.f,
               reinterpret_cast<float2*>(wsb), 0, below ? opts->below_apply_act : 0};
    rc = launch_conv_dx(g, w, dz, dx, dx_accumulate, ws2, st, below ? &bb : nullptr);
    if (rc || !below) return rc;
    return below_sums(desc, dx, opts, &bb, wsb, st);
  }
  const float* dz_eff = passthrough ? delta : dz;
  rc = launch_actbn(desc->batch, desc->out_c, p.oh * p.ow, delta, y, x_norm, act, desc->slope,
                    var, gamma, desc->bn_eps, bn, passthrough ? nullptr : dz, dgamma, db, ws, st,
                    nullptr, sums_in);
  if (rc) return rc;
  float* ws2 = reinterpret_cast<float*>(ws + p.part_bytes);
  if (!below) return launch_weights_data(g, x, w, dz_eff, dw, dx, dx_accumulate, ws2, st);
  // the sums below go with the input gradient: the two gradient kernels in turn
  rc = launch_conv_dw(g, x, dz_eff, dw, ws2, st);
  if (rc) return rc;
  char* wsb = ws + p.part_bytes + p.dw_bytes;
  BnBelow bb{opts->below_y, opts->below_x_norm, opts->below_act, opts->below_slope,
             reinterpret_cast<float2*>(wsb), 0, opts->below_apply_act};
  rc = launch_conv_dx(g, w, dz_eff, dx, dx_accumulate, ws2, st, &bb);
  if (rc) return rc;
  return below_sums(desc, dx, opts, &bb, wsb, st);
}

int cbb_conv_block_forward_workspace_size(const cbb_conv_desc* desc, size_t* bytes) {
  if (!bytes) return CBB_EINVAL;
  ConvPlan p;
  const int rc = check_desc(desc, &p);
  if (rc) return rc;
  // enough for either route (a bias keeps the forward on the general kernel, which
  // needs no scratch beyond the batch-norm partials)
  *bytes = p.part_bytes + align_up(conv_forward_workspace(make_geom(*desc), false), kAlign);
  return CBB_OK;
}

int cbb_conv_block_forward(const cbb_conv_desc* desc, const float* x, const float* w,
                           const float* bias, const float* gamma, const float* beta, float* mean,
                           float* var, float* x_norm, float* y, void* workspace,
                           size_t workspace_bytes, void* stream) {
  ConvPlan p;
  int rc = check_desc(desc, &p);
  if (rc) return rc;
  const int bn = desc->batch_normalize;
  if (!x || !w || !y || y == x) return CBB_EINVAL;
  if (bn && (!gamma || !beta || !mean || !var || !x_norm || bias)) return CBB_EINVAL;
  if (!bn && (gamma || beta || mean || var || x_norm)) return CBB_EINVAL;
  if (x_norm && (x_norm == y || x_norm == x)) return CBB_EINVAL;
  const ConvGeom g = make_geom(*desc);
  const size_t need = p.part_bytes + align_up(conv_forward_workspace(g, bias != nullptr), kAlign);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace % kAlign))
    return CBB_EWORKSPACE;
  hipStream_t st = S(stream);
  float* wsf = reinterpret_cast<float*>(static_cast<char*>(workspace) + p.part_bytes);
  if (conv_forward_first_fused(g, bn))
    return launch_conv_block_forward_first(g, x, w, bn, desc->bn_eps, desc->act, desc->slope,
                                           gamma, beta, mean, var, x_norm, y, wsf, st);
  // z goes where it is consumed: into x_norm (normalised in place) or, without BN, into y
  rc = launch_conv_forward(g, x, w, bn ? nullptr : bias, bn ? x_norm : y,
                           reinterpret_cast<float*>(static_cast<char*>(workspace) + p.part_bytes),
                           st);
  if (rc) return rc;
  return launch_bn_act_forward(desc->batch, desc->out_c, p.oh * p.ow, bn, desc->bn_eps, desc->act,
                               desc->slope, gamma, beta, mean, var, bn ? x_norm : y, y, workspace,
                               st);
}

int cbb_conv_dw_forms_dz(const cbb_conv_desc* desc) {
  const int rc = check_desc(desc, nullptr);
  if (rc) return rc;
  return desc->batch_normalize == CBB_BN_BATCH && conv_dw_forms_dz_ok(make_geom(*desc)) ? 1 : 0;
}

int cbb_conv_fused_weights_data(const cbb_conv_desc* desc) {
  const int rc = check_desc(desc, nullptr);
  if (rc) return rc;
  return conv_fused_dwdx_ok(make_geom(*desc)) ? 1 : 0;
}

int cbb_conv_backward_weights_data(const cbb_conv_desc* desc, const float* x, const float* w,
                                   const float* dz, float* dw, float* dx, int dx_accumulate,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  ConvPlan p;
  int rc = check_desc(desc, &p);
  if (rc) return rc;
  if (!x || !w || !dz || !dw) return CBB_EINVAL;
  if (dx_accumulate != 0 && dx_accumulate != 1) return CBB_EINVAL;
  if (p.total > 0 && (!workspace || workspace_bytes < p.total)) return CBB_EWORKSPACE;
  if (workspace && ((uintptr_t)workspace % kAlign)) return CBB_EWORKSPACE;
  char* ws = static_cast<char*>(workspace);
  return launch_weights_data(make_geom(*desc), x, w, dz, dw, dx, dx_accumulate,
                             reinterpret_cast<float*>(ws ? ws + p.part_bytes : nullptr),
                             S(stream));
}

int cbb_conv_act_bn_backward(const cbb_conv_desc* desc, const float* y, const float* x_norm,
                             const float* var, const float* gamma, const float* delta, float* dz,
                             float* db, float* dgamma, void* workspace, size_t workspace_bytes,
                             void* stream) {
  ConvPlan p;
  int rc = check_desc(desc, &p);
  if (rc) return rc;
  const int bn = desc->batch_normalize, act = desc->act;
  if (!delta || !db) return CBB_EINVAL;
  if (act != CBB_ACT_LINEAR && !y) return CBB_EINVAL;
  if (bn && (!x_norm || !var || !gamma || !dgamma)) return CBB_EINVAL;
  if (!bn && (x_norm || var || gamma || dgamma)) return CBB_EINVAL;
  const bool passthrough = act == CBB_ACT_LINEAR && !bn;
  if (!passthrough && !dz) return CBB_EINVAL;
  if (!workspace || workspace_bytes < p.total || ((uintptr_t)workspace % kAlign))
    return CBB_EWORKSPACE;
  return launch_actbn(desc->batch, desc->out_c, p.oh * p.ow, delta, y, x_norm, act, desc->slope,
                      var, gamma, desc->bn_eps, bn, passthrough ? nullptr : dz, dgamma, db,
                      workspace, S(stream));
}

int cbb_conv_backward_weights(const cbb_conv_desc* desc, const float* x, const float* dz,
                              float* dw, void* workspace, size_t workspace_bytes, void* stream) {
  ConvPlan p;
  int rc = check_desc(desc, &p);
  if (rc) return rc;
  if (!x || !dz || !dw) return CBB_EINVAL;
  if (p.total > 0 && (!workspace || workspace_bytes < p.total)) return CBB_EWORKSPACE;
  if (workspace && ((uintptr_t)workspace % kAlign)) return CBB_EWORKSPACE;
  char* ws = static_cast<char*>(workspace);
  return launch_conv_dw(make_geom(*desc), x, dz, dw,
                        reinterpret_cast<float*>(ws ? ws + p.part_bytes : nullptr), S(stream));
}

int cbb_conv_backward_data(const cbb_conv_desc* desc, const float* w, const float* dz, float* dx,
                           int dx_accumulate, void* workspace, size_t workspace_bytes,
                           void* stream) {
  ConvPlan p;
  int rc = check_desc(desc, &p);
  if (rc) return rc;
  if (!w || !dz || !dx) return CBB_EINVAL;
  if (dx_accumulate != 0 && dx_accumulate != 1) return CBB_EINVAL;
  if (p.total > 0 && (!workspace || workspace_bytes < p.total)) return CBB_EWORKSPACE;
  if (workspace && ((uintptr_t)workspace % kAlign)) return CBB_EWORKSPACE;
  char* ws = static_cast<char*>(workspace);
  return launch_conv_dx(make_geom(*desc), w, dz, dx, dx_accumulate,
                        reinterpret_cast<float*>(ws ? ws + p.part_bytes : nullptr), S(stream));
}

int cbb_conv_backward_data_ex(const cbb_conv_desc* desc, const float* w, const float* dz,
                              float* dx, int dx_accumulate, const cbb_block_opts* opts,
                              void* workspace, size_t workspace_bytes, void* stream) {
  ConvPlan p;
  int rc = check_desc(desc, &p);
  if (rc) return rc;
  if (!w || !dz || !dx) return CBB_EINVAL;
  if (dx_accumulate != 0 && dx_accumulate != 1) return CBB_EINVAL;
  if (opts && opts->sums) return CBB_EINVAL;   // no act/BN stage in this call
  rc = check_block_opts(desc, dx, opts);
  if (rc) return rc;
  if (p.total > 0 && (!workspace || workspace_bytes < p.total)) return CBB_EWORKSPACE;
  if (workspace && ((uintptr_t)workspace % kAlign)) return CBB_EWORKSPACE;
  char* ws = static_cast<char*>(workspace);
  const bool below = opts && opts->below_sums;
  char* wsb = ws + p.part_bytes + p.dw_bytes;
  BnBelow bb{below ? opts->below_y : nullptr, below ? opts->below_x_norm : nullptr,
             below ? opts->below_act : 0, below ? opts->below_slope : 0.f,
             reinterpret_cast<float2*>(wsb), 0, below ? opts->below_apply_act : 0};
  rc = launch_conv_dx(make_geom(*desc), w, dz, dx, dx_accumulate,
                      reinterpret_cast<float*>(ws + p.part_bytes), S(stream),
                      below ? &bb : nullptr);
  if (rc || !below) return rc;
  return below_sums(desc, dx, opts, &bb, wsb, S(stream));
}

int cbb_conv_fuses_below_sums(const cbb_conv_desc* desc) {
  const int rc = check_desc(desc, nullptr);
  if (rc) return rc;
  return conv_dx_sums_below_ok(make_geom(*desc)) ? 1 : 0;
}

int cbb_act_backward(int act, float slope, const float* y, const float* delta, float* g,
                     int64_t count, void* stream) {
  if (act < CBB_ACT_LINEAR || act > CBB_ACT_LOGGY) return CBB_EINVAL;
  if (count < 0 || !y || !delta || !g) return CBB_EINVAL;
  if (count == 0) return CBB_OK;
  return launch_act_backward(act, slope, y, delta, g, count, S(stream));
}

int cbb_bn_backward_workspace_size(int n, int c, int64_t hw, size_t* bytes) {
  if (!bytes || n < 1 || c < 1 || hw < 1) return CBB_EINVAL;
  if ((int64_t)n * c * hw >= kMaxIndex) return CBB_EUNSUPPORTED;
  *bytes = align_up(actbn_workspace(n, c, hw), kAlign);
  return CBB_OK;
}

static int bn_backward_mode(int mode, int n, int c, int64_t hw, float eps, const float* g,
                            const float* x_norm, const float* var, const float* gamma, float* dz,
                            float* dgamma, float* dbeta, void* workspace, size_t workspace_bytes,
                            void* stream) {
  size_t need = 0;
  int rc = cbb_bn_backward_workspace_size(n, c, hw, &need);
  if (rc) return rc;
  if (!(eps > 0.f) || !g || !x_norm || !var || !gamma || !dz || !dgamma || !dbeta)
    return CBB_EINVAL;
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace % kAlign))
    return CBB_EWORKSPACE;
  return launch_actbn(n, c, hw, g, nullptr, x_norm, CBB_ACT_LINEAR, 0.f, var, gamma, eps, mode, dz,
                      dgamma, dbeta, workspace, S(stream));
}

int cbb_bn_backward(int n, int c, int64_t hw, float eps, const float* g, const float* x_norm,
                    const float* var, const float* gamma, float* dz, float* dgamma, float* dbeta,
                    void* workspace, size_t workspace_bytes, void* stream) {
  return bn_backward_mode(CBB_BN_BATCH, n, c, hw, eps, g, x_norm, var, gamma, dz, dgamma, dbeta,
                          workspace, workspace_bytes, stream);
}

int cbb_bn_backward_fixed(int n, int c, int64_t hw, float eps, const float* g,
                          const float* x_norm, const float* var, const float* gamma, float* dz,
                          float* dgamma, float* dbeta, void* workspace, size_t workspace_bytes,
                          void* stream) {
  return bn_backward_mode(CBB_BN_FIXED, n, c, hw, eps, g, x_norm, var, gamma, dz, dgamma, dbeta,
                          workspace, workspace_bytes, stream);
}

int cbb_fc_backward(int batch, int in_dim, int out_dim, const float* x, const float* w,
                    const float* delta, float* dw, float* db, float* dx, int dx_accumulate,
                    void* stream) {
  if (batch < 1 || in_dim < 1 || out_dim < 1 || !x || !w || !delta || !dw) return CBB_EINVAL;
  if (dx_accumulate != 0 && dx_accumulate != 1) return CBB_EINVAL;
  if ((int64_t)batch * in_dim >= kMaxIndex || (int64_t)out_dim * in_dim >= kMaxIndex ||
      (int64_t)batch * out_dim >= kMaxIndex)
    return CBB_EUNSUPPORTED;
  return launch_fc(batch, in_dim, out_dim, x, w, delta, dw, db, dx, dx_accumulate, S(stream));
}

int cbb_softmax_loss_backward(int batch, int classes, const float* prob, const int32_t* labels,
                              float loss_weight, float* dlogits, int32_t* bad_labels,
                              void* stream) {
  if (batch < 1 || classes < 1 || !prob || !labels || !dlogits) return CBB_EINVAL;
  if ((int64_t)batch * classes >= kMaxIndex) return CBB_EUNSUPPORTED;
  return launch_softmax_loss(batch, classes, prob, labels, loss_weight, dlogits, bad_labels,
                             S(stream));
}

int cbb_fc_softmax_backward(int batch, int in_dim, int classes, const float* prob,
                            const int32_t* labels, float loss_weight, const float* x,
                            const float* w, float* dlogits, float* dw, float* db, float* dx,
                            int32_t* bad_labels, void* stream) {
  if (batch < 1 || in_dim < 1 || classes < 1 || !prob || !labels || !x || !w || !dlogits || !dw)
    return CBB_EINVAL;
  if ((int64_t)batch * in_dim >= kMaxIndex || (int64_t)classes * in_dim >= kMaxIndex ||
      (int64_t)batch * classes >= kMaxIndex)
    return CBB_EUNSUPPORTED;
  int rc = launch_softmax_loss(batch, classes, prob, labels, loss_weight, dlogits, bad_labels,
                               S(stream));
  if (rc) return rc;
  return launch_fc(batch, in_dim, classes, x, w, dlogits, dw, db, dx, 0, S(stream));
}

int cbb_softmax_backward(int outer, int channels, int64_t inner, const float* y, const float* dy,
                         float* dx, void* stream) {
  if (outer < 1 || channels < 1 || inner < 1 || !y || !dy || !dx) return CBB_EINVAL;
  if (dx == y) return CBB_EINVAL;
  if ((int64_t)outer * channels * inner >= kMaxIndex) return CBB_EUNSUPPORTED;
  return launch_softmax_backward(outer, channels, inner, y, dy, dx, S(stream));
}

int cbb_shortcut_backward_resize(int batch, int w1, int h1, int c1, int w2, int h2, int c2,
                                 float alpha, float beta, const float* delta, float* d_main,
                                 float* d_from, void* stream) {
  if (batch < 1 || w1 < 1 || h1 < 1 || c1 < 1 || w2 < 1 || h2 < 1 || c2 < 1 || !delta || !d_from)
    return CBB_EINVAL;
  if (d_from == delta || d_main == delta || (d_main && d_main == d_from)) return CBB_EINVAL;
  // the page's asserts: one integer ratio for both sides, the same aspect
  if (w1 / w2 != h1 / h2 || w2 / w1 != h2 / h1) return CBB_ESHAPE;
  if ((int64_t)batch * c1 * h1 * w1 >= kMaxIndex || (int64_t)batch * c2 * h2 * w2 >= kMaxIndex)
    return CBB_EUNSUPPORTED;
  return launch_shortcut_resize(batch, w1, h1, c1, w2, h2, c2, alpha, beta, delta, d_main, d_from,
                                S(stream));
}

int cbb_shortcut_backward(int64_t count, float alpha, float beta, const float* delta,
                          float* d_main, float* d_from, void* stream) {
  if (count < 0 || !delta || !d_main || !d_from) return CBB_EINVAL;
  if (d_main == d_from || d_main == delta || d_from == delta) return CBB_EINVAL;
  if (count == 0) return CBB_OK;
  return launch_shortcut(count, alpha, beta, delta, d_main, d_from, S(stream));
}

int cbb_route_backward(int batch, int n_in, const int64_t* in_sizes, const float* delta,
                       float* const* d_in, void* stream) {
  if (batch < 1 || n_in < 1 || n_in > 8 || !in_sizes || !delta || !d_in) return CBB_EINVAL;
  int64_t outputs = 0;
  for (int t = 0; t < n_in; ++t) {
    if (in_sizes[t] < 1 || !d_in[t]) return CBB_EINVAL;
    outputs += in_sizes[t];
  }
  if (outputs * batch >= kMaxIndex) return CBB_EUNSUPPORTED;
  return launch_route(batch, n_in, in_sizes, delta, d_in, S(stream));
}

int cbb_upsample_backward(int n, int c, int h, int w, int scale, const float* delta, float* dx,
                          void* stream) {
  if (n < 1 || c < 1 || h < 1 || w < 1 || scale < 1 || !delta || !dx) return CBB_EINVAL;
  if (scale > 8) return CBB_EUNSUPPORTED;
  if ((int64_t)n * c * h * w * scale * scale >= kMaxIndex) return CBB_EUNSUPPORTED;
  return launch_upsample(n, c, h, w, scale, delta, dx, S(stream));
}

int cbb_sgd_update(int64_t n, int batch, float learning_rate, float momentum, float decay,
                   float* w, float* dw, void* stream) {
  if (n < 0 || batch < 1 || !w || !dw || w == dw) return CBB_EINVAL;
  if (!(learning_rate >= 0.f) || !(momentum >= 0.f) || !(decay >= 0.f)) return CBB_EINVAL;
  if (n == 0) return CBB_OK;
  return launch_sgd_update(n, batch, learning_rate, momentum, decay, w, dw, S(stream));
}

int cbb_maxpool_backward(int n, int c, int ih, int iw, int ksize, int stride,
                         const int32_t* idx, const float* delta, float* dx, void* stream) {
  if (n < 1 || c < 1 || ih < 1 || iw < 1 || ksize < 1 || stride < 1 || !idx || !delta || !dx)
    return CBB_EINVAL;
  if (ksize > ih || ksize > iw) return CBB_ESHAPE;
  if ((int64_t)n * c * ih * iw >= kMaxIndex) return CBB_EUNSUPPORTED;
  return launch_maxpool(n, c, ih, iw, ksize, stride, idx, delta, dx, S(stream));
}

}  // extern "C"
