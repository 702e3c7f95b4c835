// C ABI of libskiparse: argument validation, the host plan, and dispatch to
// the HIP kernels.  See include/skiparse.h for the contract of each call.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "block.h"

using namespace skiparse;

namespace {

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

constexpr float kE4M3MaxHost = 448.0f;

int ok() {
  g_err.clear();
  return SKIPARSE_OK;
}

// Real local extent on one axis of stride k for coordinate p (any-resolution
// rule: the real members are a prefix of the local axis); rule 0 token-wise,
// 1 group-wise.
int32_t real_extent(int32_t n, int32_t k, int32_t rule, int32_t p) {
  if (k == 1) return n;
  if (rule == 0) return n / k + (p < n % k ? 1 : 0);
  const int32_t kk = k * k;
  int32_t r = n % kk - p * k;
  r = r < 0 ? 0 : (r > k ? k : r);
  return (n / kk) * k + r;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

// Re-derive a plan from its inputs and compare, so a hand-edited or stale
// struct is refused instead of driving the kernels out of bounds.
int check_plan(const skiparse_plan* p) {
  if (!p) return fail(SKIPARSE_EINVAL, "plan is NULL");
  if (p->abi != SKIPARSE_ABI_VERSION) return fail(SKIPARSE_EINVAL, "plan has ABI %d, library %d", p->abi, SKIPARSE_ABI_VERSION);
  skiparse_plan q;
  const std::string saved = g_err;
  if (skiparse_plan_init(&q, p->B, p->T, p->H, p->W, p->heads, p->d, p->k, p->mode) != SKIPARSE_OK)
    return fail(SKIPARSE_EINVAL, "plan fields are invalid: %s", g_err.c_str());
  if (std::memcmp(&q, p, sizeof q) != 0) return fail(SKIPARSE_EINVAL, "plan was modified after skiparse_plan_init");
  g_err = saved;
  return SKIPARSE_OK;
}

bool is_1d(int32_t mode) { return mode == SKIPARSE_MODE_TOKEN_1D || mode == SKIPARSE_MODE_GROUP_1D; }

// Strides along the kernels' h and w axes.  Skiparse-1D runs along each
// frame's flattened l = h*W + w (grid (T, 1, H*W)) with stride k*k.
int32_t stride_h(const skiparse_plan& p) { return is_1d(p.mode) ? 1 : p.k; }
int32_t stride_w(const skiparse_plan& p) { return is_1d(p.mode) ? p.k * p.k : p.k; }

void make_geom(const skiparse_plan& p, Geom& g) {
  g.T = p.T;
  g.H = is_1d(p.mode) ? 1 : p.H;
  g.W = is_1d(p.mode) ? p.H * p.W : p.W;
  g.kh = stride_h(p);
  g.kw = stride_w(p);
  g.rule = (p.mode == SKIPARSE_MODE_GROUP || p.mode == SKIPARSE_MODE_GROUP_1D) ? 1 : 0;
  g.div_kh = make_fastdiv((uint32_t)g.kh);
  g.div_kw = make_fastdiv((uint32_t)g.kw);
}

SubGeom make_sub(const skiparse_plan& p, int s) {
  SubGeom sg;
  const int kw = stride_w(p);
  const int pp = s / kw, qq = s % kw;
  const int32_t hr = p.real_h[pp], wr = p.real_w[qq];
  sg.n = p.T * hr * wr;
  sg.p = pp;
  sg.q = qq;
  sg.tile0 = 0;
  sg.div_hw = make_fastdiv((uint32_t)(hr * wr > 0 ? hr * wr : 1));
  sg.div_w = make_fastdiv((uint32_t)(wr > 0 ? wr : 1));
  if (hr * wr == 0) {   // keep the stored extents exact for the map writer
    sg.div_hw.d = (uint32_t)(hr * wr);
    sg.div_w.d = (uint32_t)wr;
    sg.n = 0;
  }
  return sg;
}

// Range and scale checks shared by the entry points that run the attention;
// fills the call-wide part of AttnArgs (geometry, subsequences, scale) and
// leaves every pointer NULL.
int fill_attn_args(const skiparse_plan* plan, float softmax_scale, int32_t sub_begin, int32_t& sub_count,
                   AttnArgs& a) {
  if (sub_count == 0) {
    if (sub_begin != 0) return fail(SKIPARSE_EINVAL, "sub_count == 0 (all) needs sub_begin == 0");
    sub_count = plan->n_sub;
  }
  // compared without forming sub_begin + sub_count, which can overflow int32
  if (sub_begin < 0 || sub_count < 0 || sub_begin > plan->n_sub || sub_count > plan->n_sub - sub_begin)
    return fail(SKIPARSE_EINVAL, "subsequence range [%d, %lld) outside [0, %d)", sub_begin,
                (long long)sub_begin + sub_count, plan->n_sub);
  if (!(std::isfinite(softmax_scale))) return fail(SKIPARSE_EINVAL, "softmax_scale must be finite");
  const int d = plan->d;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)d);
  std::memset(&a, 0, sizeof a);
  a.batch_stride = (int64_t)plan->T * plan->H * plan->W * plan->heads * d;
  a.row_stride = plan->heads * d;
  a.heads = plan->heads;
  a.n_run = sub_count;
  a.scale = scale;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  make_geom(*plan, a.g);
  for (int i = 0; i < sub_count; ++i) a.sub[i] = make_sub(*plan, sub_begin + i);
  return SKIPARSE_OK;
}

// The training entry points: bf16 only, then the common part.
int training_args(const skiparse_plan* plan, skiparse_dtype dtype, float softmax_scale, int32_t sub_begin,
                  int32_t& sub_count, AttnArgs& a) {
  if (dtype != SKIPARSE_BF16) return fail(SKIPARSE_EUNSUPPORTED, "training calls are built for BF16 only");
  return fill_attn_args(plan, softmax_scale, sub_begin, sub_count, a);
}

}  // namespace

extern "C" {

int skiparse_abi_version(void) { return SKIPARSE_ABI_VERSION; }

const char* skiparse_last_error(void) { return g_err.c_str(); }

int skiparse_plan_init(skiparse_plan* plan, int32_t B, int32_t T, int32_t H, int32_t W, int32_t heads,
                       int32_t d, int32_t k, int32_t mode) {
  if (!plan) return fail(SKIPARSE_EINVAL, "plan is NULL");
  if (B < 1 || T < 1 || H < 1 || W < 1 || heads < 1 || d < 1)
    return fail(SKIPARSE_EINVAL, "every extent must be >= 1 (B=%d T=%d H=%d W=%d heads=%d d=%d)", B, T, H, W, heads, d);
  if (k < 1 || k > SKIPARSE_MAX_K) return fail(SKIPARSE_EINVAL, "k=%d outside [1, %d]", k, SKIPARSE_MAX_K);
  if (mode < SKIPARSE_MODE_TOKEN || mode > SKIPARSE_MODE_GROUP_1D)
    return fail(SKIPARSE_EINVAL, "mode=%d is not token (0), group (1), token-1D (2) or group-1D (3)", mode);
  const bool one_d = k > 1 && (mode == SKIPARSE_MODE_TOKEN_1D || mode == SKIPARSE_MODE_GROUP_1D);
  if (one_d && k * k > SKIPARSE_MAX_K)
    return fail(SKIPARSE_EINVAL, "the 1-D modes hold k*k subsequences in the plan's real_w[%d]: k <= 2 (k=%d)", SKIPARSE_MAX_K, k);
  const int64_t kk = (int64_t)k * k;
  // the grid the pattern runs on: (T, H, W), or (T, 1, H*W) for Skiparse-1D
  const int64_t gh = one_d ? 1 : H, gw = one_d ? (int64_t)H * W : W;
  const int64_t sh = one_d ? 1 : k, swd = one_d ? kk : k;   // strides along the grid's axes
  const int64_t Hp = (gh + sh * sh - 1) / (sh * sh) * (sh * sh), Wp = (gw + swd * swd - 1) / (swd * swd) * (swd * swd);
  const int64_t tokens = (int64_t)T * H * W;
  const int64_t padded = (int64_t)T * Hp * Wp;
  if (padded >= (int64_t(1) << 31)) return fail(SKIPARSE_EINVAL, "T*Hp*Wp = %lld must stay below 2^31", (long long)padded);
  const double numel = (double)B * tokens * heads * d;
  if (numel >= 4.6e18 || (int64_t)heads * d >= (int64_t(1) << 31))
    return fail(SKIPARSE_EINVAL, "tensor too large");
  std::memset(plan, 0, sizeof *plan);
  plan->abi = SKIPARSE_ABI_VERSION;
  plan->B = B;
  plan->T = T;
  plan->H = H;
  plan->W = W;
  plan->heads = heads;
  plan->d = d;
  plan->k = k;
  plan->mode = k == 1 ? SKIPARSE_MODE_TOKEN : mode;
  plan->Hp = (int32_t)Hp;
  plan->Wp = (int32_t)Wp;
  plan->sub_h = (int32_t)(Hp / sh);
  plan->sub_w = (int32_t)(Wp / swd);
  plan->n_sub = (int32_t)kk;
  plan->sub_len_padded = (int64_t)T * plan->sub_h * plan->sub_w;
  const int32_t rule = (plan->mode == SKIPARSE_MODE_GROUP || plan->mode == SKIPARSE_MODE_GROUP_1D) ? 1 : 0;
  for (int p = 0; p < sh; ++p) plan->real_h[p] = real_extent((int32_t)gh, (int32_t)sh, rule, p);
  for (int q = 0; q < swd; ++q) plan->real_w[q] = real_extent((int32_t)gw, (int32_t)swd, rule, q);
  double pairs = 0;
  int64_t pairs_i = 0;
  for (int p = 0; p < sh; ++p)
    for (int q = 0; q < swd; ++q) {
      const int64_t n = (int64_t)T * plan->real_h[p] * plan->real_w[q];
      pairs += (double)n * n;
      pairs_i += n * n;
    }
  if (pairs * B * heads >= 9.0e18) return fail(SKIPARSE_EINVAL, "pair count overflows int64");
  plan->pairs = pairs_i * B * heads;
  return ok();
}

int skiparse_plan_index_map(const skiparse_plan* plan, int32_t* host_gather) {
  if (int e = check_plan(plan)) return e;
  if (!host_gather) return fail(SKIPARSE_EINVAL, "host_gather is NULL");
  Geom g;
  make_geom(*plan, g);
  const int64_t L = plan->sub_len_padded;
  for (int s = 0; s < plan->n_sub; ++s) {
    const SubGeom sg = make_sub(*plan, s);
    const int32_t kw = stride_w(*plan);
    const int32_t hr = plan->real_h[s / kw], wr = plan->real_w[s % kw];
    int32_t* row = host_gather + (int64_t)s * L;
    int64_t x = 0;
    for (int32_t t = 0; t < plan->T; ++t)
      for (int32_t hl = 0; hl < plan->sub_h; ++hl)
        for (int32_t wl = 0; wl < plan->sub_w; ++wl, ++x) {
          if (hl < hr && wl < wr) {
            const uint32_t j = ((uint32_t)t * hr + hl) * (uint32_t)wr + wl;
            row[x] = (int32_t)token_of(j, sg, g);
          } else {
            row[x] = -1;
          }
        }
  }
  return ok();
}

int skiparse_index_map_device(const skiparse_plan* plan, int32_t* dev_gather, hipStream_t stream) {
  if (int e = check_plan(plan)) return e;
  if (!dev_gather) return fail(SKIPARSE_EINVAL, "dev_gather is NULL");
  if (((uintptr_t)dev_gather & 3u) != 0) return fail(SKIPARSE_EINVAL, "dev_gather must be 4-byte aligned");
  Geom g;
  make_geom(*plan, g);
  SubGeom subs[kMaxRun];
  for (int s = 0; s < plan->n_sub; ++s) subs[s] = make_sub(*plan, s);
  (void)hipGetLastError();
  const hipError_t e = launch_index_map(g, subs, plan->n_sub, plan->sub_h, plan->sub_w, dev_gather, stream);
  if (e != hipSuccess) return fail(SKIPARSE_EHIP, "index map launch failed: %s", hipGetErrorString(e));
  return ok();
}

int skiparse_attn_fwd(const skiparse_plan* plan, skiparse_dtype dtype, const void* q, const void* k, const void* v,
                      void* o, float softmax_scale, const float* dev_descale_qkv, int32_t sub_begin,
                      int32_t sub_count, hipStream_t stream) {
  if (int e = check_plan(plan)) return e;
  const int d = plan->d;
  size_t in_elt, out_elt;
  switch (dtype) {
    case SKIPARSE_F32: in_elt = 4; out_elt = 4; break;
    case SKIPARSE_BF16: in_elt = 2; out_elt = 2; break;
    case SKIPARSE_FP8_E4M3: in_elt = 1; out_elt = 2; break;
    default: return fail(SKIPARSE_EINVAL, "unknown dtype %d", (int)dtype);
  }
  if (dtype == SKIPARSE_FP8_E4M3) {
    if (d != 128) return fail(SKIPARSE_EUNSUPPORTED, "FP8 attention is built for d=128 only (d=%d)", d);
    if (!dev_descale_qkv) return fail(SKIPARSE_EINVAL, "FP8 needs dev_descale_qkv");
    if (((uintptr_t)dev_descale_qkv & 3u) != 0) return fail(SKIPARSE_EINVAL, "dev_descale_qkv must be 4-byte aligned");
  } else {
    if (d != 64 && d != 128) return fail(SKIPARSE_EUNSUPPORTED, "d=%d is not built (64 or 128)", d);
    if (dev_descale_qkv) return fail(SKIPARSE_EINVAL, "dev_descale_qkv must be NULL unless dtype is FP8");
  }
  if (!q || !k || !v || !o) return fail(SKIPARSE_EINVAL, "q, k, v and o must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(SKIPARSE_EINVAL, "q, k, v and o must be 16-byte aligned");
  const int64_t numel = (int64_t)plan->B * plan->T * plan->H * plan->W * plan->heads * d;
  if (overlap(o, numel * out_elt, q, numel * in_elt) || overlap(o, numel * out_elt, k, numel * in_elt) ||
      overlap(o, numel * out_elt, v, numel * in_elt))
    return fail(SKIPARSE_EINVAL, "o must not overlap q, k or v");
  AttnArgs a;
  if (int e = fill_attn_args(plan, softmax_scale, sub_begin, sub_count, a)) return e;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.descale = dev_descale_qkv;

  (void)hipGetLastError();   // drop an error left by unrelated earlier work
  hipError_t e;
  switch (dtype) {
    case SKIPARSE_F32: e = launch_attn_f32(a, plan->B, d, stream); break;
    case SKIPARSE_BF16: e = launch_attn_bf16(a, plan->B, d, stream); break;
    default: e = launch_attn_fp8(a, plan->B, d, stream); break;
  }
  if (e == hipErrorNotSupported) return fail(SKIPARSE_EUNSUPPORTED, "this dtype has no kernel in the library");
  if (e != hipSuccess) return fail(SKIPARSE_EHIP, "attention launch failed: %s", hipGetErrorString(e));
  return ok();
}

namespace {

int64_t row_count(const skiparse_plan* plan) { return (int64_t)plan->B * plan->T * plan->H * plan->W * plan->heads; }

}  // namespace

int skiparse_attn_fwd_lse(const skiparse_plan* plan, skiparse_dtype dtype, const void* q, const void* k,
                          const void* v, void* o, float* lse, float softmax_scale, int32_t sub_begin,
                          int32_t sub_count, hipStream_t stream) {
  if (int e = check_plan(plan)) return e;
  AttnArgs a;
  if (int e = training_args(plan, dtype, softmax_scale, sub_begin, sub_count, a)) return e;
  const int d = plan->d;
  if (d != 64 && d != 128) return fail(SKIPARSE_EUNSUPPORTED, "d=%d is not built (64 or 128)", d);
  if (!q || !k || !v || !o || !lse) return fail(SKIPARSE_EINVAL, "q, k, v, o and lse must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(SKIPARSE_EINVAL, "q, k, v and o must be 16-byte aligned");
  if (((uintptr_t)lse & 3u) != 0) return fail(SKIPARSE_EINVAL, "lse must be 4-byte aligned");
  const int64_t bytes = row_count(plan) * d * 2;
  const int64_t lbytes = row_count(plan) * 4;
  if (overlap(o, bytes, q, bytes) || overlap(o, bytes, k, bytes) || overlap(o, bytes, v, bytes))
    return fail(SKIPARSE_EINVAL, "o must not overlap q, k or v");
  if (overlap(lse, lbytes, q, bytes) || overlap(lse, lbytes, k, bytes) || overlap(lse, lbytes, v, bytes) ||
      overlap(lse, lbytes, o, bytes))
    return fail(SKIPARSE_EINVAL, "lse must not overlap q, k, v or o");
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  (void)hipGetLastError();
  const hipError_t e = launch_attn_bf16(a, plan->B, d, stream);
  if (e != hipSuccess) return fail(SKIPARSE_EHIP, "attention launch failed: %s", hipGetErrorString(e));
  return ok();
}

size_t skiparse_attn_bwd_workspace_bytes(const skiparse_plan* plan) {
  if (check_plan(plan)) return 0;
  return (size_t)row_count(plan) * sizeof(float);
}

int skiparse_attn_bwd(const skiparse_plan* plan, skiparse_dtype dtype, const void* q, const void* k, const void* v,
                      const void* o, const void* dout, const float* lse, void* dq, void* dk, void* dv,
                      float softmax_scale, void* workspace, size_t workspace_bytes, int32_t sub_begin,
                      int32_t sub_count, hipStream_t stream) {
  if (int e = check_plan(plan)) return e;
  AttnArgs a;
  if (int e = training_args(plan, dtype, softmax_scale, sub_begin, sub_count, a)) return e;
  const int d = plan->d;
  if (d != 128) return fail(SKIPARSE_EUNSUPPORTED, "the backward pass is built for d=128 only (d=%d)", d);
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv)
    return fail(SKIPARSE_EINVAL, "q, k, v, o, dout, lse, dq, dk and dv must be non-NULL");
  for (const void* x : {q, k, v, o, dout, (const void*)dq, (const void*)dk, (const void*)dv})
    if (!aligned16(x)) return fail(SKIPARSE_EINVAL, "q, k, v, o, dout, dq, dk and dv must be 16-byte aligned");
  if (((uintptr_t)lse & 3u) != 0) return fail(SKIPARSE_EINVAL, "lse must be 4-byte aligned");
  const size_t need = skiparse_attn_bwd_workspace_bytes(plan);
  if (!workspace || workspace_bytes < need)
    return fail(SKIPARSE_EWORKSPACE, "workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
  if (((uintptr_t)workspace & 3u) != 0) return fail(SKIPARSE_EINVAL, "workspace must be 4-byte aligned");
  const int64_t bytes = row_count(plan) * d * 2;
  const int64_t lbytes = row_count(plan) * 4;
  const void* ins[] = {q, k, v, o, dout};
  const int64_t insz[] = {bytes, bytes, bytes, bytes, bytes};
  void* outs[] = {dq, dk, dv, workspace};
  const int64_t outsz[] = {bytes, bytes, bytes, (int64_t)need};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 5; ++j)
      if (overlap(outs[i], outsz[i], ins[j], insz[j])) return fail(SKIPARSE_EINVAL, "outputs and workspace must not overlap the inputs");
    if (overlap(outs[i], outsz[i], lse, lbytes)) return fail(SKIPARSE_EINVAL, "outputs and workspace must not overlap lse");
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outsz[i], outs[j], outsz[j])) return fail(SKIPARSE_EINVAL, "dq, dk, dv and workspace must not overlap");
  }
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = const_cast<void*>(o);   // read only by the backward kernels
  a.dout = dout;
  a.lse = const_cast<float*>(lse);
  a.dsum = (float*)workspace;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  (void)hipGetLastError();
  const hipError_t e = launch_attn_bwd(a, plan->B, d, stream);
  if (e == hipErrorNotSupported) return fail(SKIPARSE_EUNSUPPORTED, "this head dim has no backward kernel in the library");
  if (e != hipSuccess) return fail(SKIPARSE_EHIP, "backward launch failed: %s", hipGetErrorString(e));
  return ok();
}

int skiparse_attn_fwd_lse_fp8(const skiparse_plan* plan, const void* q8, const void* k8, const void* v8,
                              const float* dev_descale_qkv, void* o, float* lse, float softmax_scale,
                              int32_t sub_begin, int32_t sub_count, hipStream_t stream) {
  if (int e = check_plan(plan)) return e;
  const int d = plan->d;
  if (d != 128) return fail(SKIPARSE_EUNSUPPORTED, "FP8 attention is built for d=128 only (d=%d)", d);
  if (!q8 || !k8 || !v8 || !dev_descale_qkv || !o || !lse)
    return fail(SKIPARSE_EINVAL, "q8, k8, v8, dev_descale_qkv, o and lse must be non-NULL");
  if (!aligned16(q8) || !aligned16(k8) || !aligned16(v8) || !aligned16(o))
    return fail(SKIPARSE_EINVAL, "q8, k8, v8 and o must be 16-byte aligned");
  if ((((uintptr_t)lse | (uintptr_t)dev_descale_qkv) & 3u) != 0)
    return fail(SKIPARSE_EINVAL, "lse and dev_descale_qkv must be 4-byte aligned");
  const int64_t n8 = row_count(plan) * d, nl = row_count(plan) * 4;
  const void* ins[] = {q8, k8, v8, dev_descale_qkv};
  const int64_t insz[] = {n8, n8, n8, 6 * 4};
  for (int j = 0; j < 4; ++j)
    if (overlap(o, n8 * 2, ins[j], insz[j]) || overlap(lse, nl, ins[j], insz[j]))
      return fail(SKIPARSE_EINVAL, "o and lse must not overlap q8, k8, v8 or dev_descale_qkv");
  if (overlap(o, n8 * 2, lse, nl)) return fail(SKIPARSE_EINVAL, "lse must not overlap o");
  AttnArgs a;
  if (int e = fill_attn_args(plan, softmax_scale, sub_begin, sub_count, a)) return e;
  a.q = q8;
  a.k = k8;
  a.v = v8;
  a.o = o;
  a.lse = lse;
  a.descale = dev_descale_qkv;
  (void)hipGetLastError();
  const hipError_t e = launch_attn_fp8(a, plan->B, d, stream);
  if (e != hipSuccess) return fail(SKIPARSE_EHIP, "attention launch failed: %s", hipGetErrorString(e));
  return ok();
}

int skiparse_attn_bwd_fp8(const skiparse_plan* plan, const void* q8, const void* k8, const void* v8,
                          const float* dev_descale_qkv, const void* o, const void* dout8,
                          const float* dev_descale_dout, const float* lse, void* dq, void* dk, void* dv,
                          float softmax_scale, void* workspace, size_t workspace_bytes, int32_t sub_begin,
                          int32_t sub_count, hipStream_t stream) {
  if (int e = check_plan(plan)) return e;
  const int d = plan->d;
  if (d != 128) return fail(SKIPARSE_EUNSUPPORTED, "the backward pass is built for d=128 only (d=%d)", d);
  if (!q8 || !k8 || !v8 || !dev_descale_qkv || !o || !dout8 || !dev_descale_dout || !lse || !dq || !dk || !dv)
    return fail(SKIPARSE_EINVAL,
                "q8, k8, v8, dev_descale_qkv, o, dout8, dev_descale_dout, lse, dq, dk and dv must be non-NULL");
  for (const void* x : {q8, k8, v8, o, dout8, (const void*)dq, (const void*)dk, (const void*)dv})
    if (!aligned16(x)) return fail(SKIPARSE_EINVAL, "q8, k8, v8, o, dout8, dq, dk and dv must be 16-byte aligned");
  if ((((uintptr_t)lse | (uintptr_t)dev_descale_qkv | (uintptr_t)dev_descale_dout) & 3u) != 0)
    return fail(SKIPARSE_EINVAL, "lse, dev_descale_qkv and dev_descale_dout must be 4-byte aligned");
  const size_t need = skiparse_attn_bwd_workspace_bytes(plan);
  if (!workspace || workspace_bytes < need)
    return fail(SKIPARSE_EWORKSPACE, "workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
  if (((uintptr_t)workspace & 3u) != 0) return fail(SKIPARSE_EINVAL, "workspace must be 4-byte aligned");
  const int64_t n8 = row_count(plan) * d, nl = row_count(plan) * 4;
  const void* ins[] = {q8, k8, v8, dev_descale_qkv, o, dout8, dev_descale_dout, lse};
  const int64_t insz[] = {n8, n8, n8, 6 * 4, n8 * 2, n8, 2 * 4, nl};
  void* outs[] = {dq, dk, dv, workspace};
  const int64_t outsz[] = {n8 * 2, n8 * 2, n8 * 2, (int64_t)need};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 8; ++j)
      if (overlap(outs[i], outsz[i], ins[j], insz[j]))
        return fail(SKIPARSE_EINVAL, "outputs and workspace must not overlap the inputs, the scales or lse");
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outsz[i], outs[j], outsz[j])) return fail(SKIPARSE_EINVAL, "dq, dk, dv and workspace must not overlap");
  }
  AttnArgs a;
  if (int e = fill_attn_args(plan, softmax_scale, sub_begin, sub_count, a)) return e;
  a.q = q8;
  a.k = k8;
  a.v = v8;
  a.descale = dev_descale_qkv;
  a.o = const_cast<void*>(o);   // read only by the backward kernels
  a.dout = dout8;
  a.descale_do = dev_descale_dout;
  a.lse = const_cast<float*>(lse);
  a.dsum = (float*)workspace;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  (void)hipGetLastError();
  const hipError_t e = launch_attn_bwd_fp8(a, plan->B, d, stream);
  if (e != hipSuccess) return fail(SKIPARSE_EHIP, "backward launch failed: %s", hipGetErrorString(e));
  return ok();
}

size_t skiparse_quant_fp8_workspace_bytes(int64_t numel) { return quant_workspace_bytes(numel < 0 ? 0 : numel); }

int skiparse_quant_fp8(const void* x, skiparse_dtype x_dtype, int64_t numel, uint8_t* y, float* dev_scale,
                       float fp8_max, float eps, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (x_dtype != SKIPARSE_BF16 && x_dtype != SKIPARSE_F32)
    return fail(SKIPARSE_EINVAL, "x_dtype must be BF16 or F32");
  if (numel < 1) return fail(SKIPARSE_EINVAL, "numel must be >= 1");
  if (!x || !y || !dev_scale) return fail(SKIPARSE_EINVAL, "x, y and dev_scale must be non-NULL");
  if (!aligned16(x) || !aligned16(y) || ((uintptr_t)dev_scale & 3u) != 0)
    return fail(SKIPARSE_EINVAL, "x and y must be 16-byte aligned, dev_scale 4-byte aligned");
  if (!(fp8_max > 0.f) || !std::isfinite(fp8_max) || !(eps >= 0.f) || !std::isfinite(eps))
    return fail(SKIPARSE_EINVAL, "fp8_max must be positive and eps non-negative, both finite");
  const size_t need = quant_workspace_bytes(numel);
  if (!workspace || workspace_bytes < need)
    return fail(SKIPARSE_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : 0);
  if (((uintptr_t)workspace & 3u) != 0) return fail(SKIPARSE_EINVAL, "workspace must be 4-byte aligned");
  const size_t xb = (size_t)numel * (x_dtype == SKIPARSE_BF16 ? 2 : 4);
  if (overlap(y, (size_t)numel, x, xb) || overlap(workspace, need, x, xb) || overlap(workspace, need, y, (size_t)numel))
    return fail(SKIPARSE_EINVAL, "x, y and workspace must not overlap");
  (void)hipGetLastError();
  const hipError_t e = launch_quant_fp8(x, x_dtype == SKIPARSE_BF16, numel, y, dev_scale, fp8_max, eps, workspace, stream);
  if (e != hipSuccess) return fail(SKIPARSE_EHIP, "quantization launch failed: %s", hipGetErrorString(e));
  return ok();
}

int skiparse_quant_fp8_noalloc(const void* x, skiparse_dtype x_dtype, int64_t numel, uint8_t* y, float* dev_scale,
                               float fp8_max, float eps, hipStream_t stream) {
  if (x_dtype != SKIPARSE_BF16 && x_dtype != SKIPARSE_F32)
    return fail(SKIPARSE_EINVAL, "x_dtype must be BF16 or F32");
  if (numel < 1) return fail(SKIPARSE_EINVAL, "numel must be >= 1");
  if (!x || !y || !dev_scale) return fail(SKIPARSE_EINVAL, "x, y and dev_scale must be non-NULL");
  if (!aligned16(x) || !aligned16(y) || ((uintptr_t)dev_scale & 3u) != 0)
    return fail(SKIPARSE_EINVAL, "x and y must be 16-byte aligned, dev_scale 4-byte aligned");
  if (!(fp8_max > 0.f) || !std::isfinite(fp8_max) || !(eps >= 0.f) || !std::isfinite(eps))
    return fail(SKIPARSE_EINVAL, "fp8_max must be positive and eps non-negative, both finite");
  const size_t need = quant_workspace_bytes(numel);
  if (need > quant_scratch_bytes())
    return fail(SKIPARSE_EWORKSPACE, "numel=%lld needs %zu bytes of scratch, above the %zu the library holds",
                (long long)numel, need, quant_scratch_bytes());
  const size_t xb = (size_t)numel * (x_dtype == SKIPARSE_BF16 ? 2 : 4);
  if (overlap(y, (size_t)numel, x, xb) || overlap(dev_scale, 8, x, xb) || overlap(dev_scale, 8, y, (size_t)numel))
    return fail(SKIPARSE_EINVAL, "x, y and dev_scale must not overlap");
  float* ws = nullptr;
  hipError_t e = quant_scratch(&ws);
  if (e != hipSuccess) return fail(SKIPARSE_EHIP, "scratch lookup failed: %s", hipGetErrorString(e));
  (void)hipGetLastError();
  e = launch_quant_fp8(x, x_dtype == SKIPARSE_BF16, numel, y, dev_scale, fp8_max, eps, ws, stream);
  if (e != hipSuccess) return fail(SKIPARSE_EHIP, "quantization launch failed: %s", hipGetErrorString(e));
  return ok();
}

// ---------------------------------------------------------------------------
// fp8 attention block
// ---------------------------------------------------------------------------

namespace {

size_t round256(size_t n) { return (n + 255) & ~size_t(255); }

// Byte offsets of the block's scratch buffers inside the caller's workspace.
struct BlockLayout {
  size_t x8, qkv16, qkv8, scales, part, tab, total;
};

// Rotary geometry of a plan's (B, T, H, W, heads, d) tensor; validates theta,
// the split and the size.
int rope_setup(const skiparse_plan& p, float theta, const int32_t* rope_dims, RopeGeom& r) {
  const int d = p.d;
  if (d < 8 || (d & (d - 1)) != 0) return fail(SKIPARSE_EUNSUPPORTED, "the rotary kernels need d a power of two >= 8 (d=%d)", d);
  if (!(theta > 0.f) || !std::isfinite(theta)) return fail(SKIPARSE_EINVAL, "rope_theta must be positive and finite");
  int32_t dims[3];
  if (rope_dims && (rope_dims[0] || rope_dims[1] || rope_dims[2])) {
    for (int i = 0; i < 3; ++i) dims[i] = rope_dims[i];
    if (dims[0] < 0 || dims[1] < 0 || dims[2] < 0 || ((dims[0] | dims[1] | dims[2]) & 1) ||
        (int64_t)dims[0] + dims[1] + dims[2] != d)
      return fail(SKIPARSE_EINVAL, "rope_dims (%d, %d, %d) must be even, non-negative and sum to d=%d", dims[0],
                  dims[1], dims[2], d);
  } else {
    dims[1] = dims[2] = 2 * (d / 6);
    dims[0] = d - 2 * dims[1];
  }
  const int64_t mc = (int64_t)p.B * p.T * p.H * p.W * p.heads * d;
  if (mc / 8 >= (int64_t(1) << 31)) return fail(SKIPARSE_EINVAL, "B*T*H*W*heads*d / 8 must stay below 2^31");
  r.T = p.T;
  r.H = p.H;
  r.W = p.W;
  r.d = d;
  r.dt = dims[0];
  r.dh = dims[1];
  r.dw = dims[2];
  r.tab_h = p.T * (dims[0] / 2);
  r.tab_w = r.tab_h + p.H * (dims[1] / 2);
  r.tab_len = r.tab_w + p.W * (dims[2] / 2);
  r.nvec = (uint32_t)(mc / 8);
  r.div_cv = make_fastdiv((uint32_t)((int64_t)p.heads * d / 8));
  r.div_w = make_fastdiv((uint32_t)p.W);
  r.div_h = make_fastdiv((uint32_t)p.H);
  r.div_t = make_fastdiv((uint32_t)p.T);
  return SKIPARSE_OK;
}

size_t rope_table_bytes(const skiparse_plan& p) {
  return round256((size_t)(p.T + p.H + p.W) * (p.d / 2) * sizeof(float2));
}

size_t rope_part_bytes(const skiparse_plan& p) {
  const size_t nvec = (size_t)p.B * p.T * p.H * p.W * p.heads * p.d / 8;
  return round256(rope_partials_bytes((uint32_t)(nvec < (size_t(1) << 31) ? nvec : 1)));
}

BlockLayout block_layout(const skiparse_plan& p) {
  const size_t mc = (size_t)p.B * p.T * p.H * p.W * p.heads * p.d;
  const size_t nvec = mc / 8;
  size_t part = quant_workspace_bytes((int64_t)mc);
  const size_t rp = rope_partials_bytes((uint32_t)(nvec < (size_t(1) << 31) ? nvec : 1));
  if (rp > part) part = rp;
  BlockLayout L;
  size_t at = 0;
  L.x8 = at, at += round256(mc);                 // x codes, later O codes
  L.qkv16 = at, at += round256(3 * mc * 2);      // Q, K, V projections (bf16), later O (bf16) over Q
  L.qkv8 = at, at += round256(3 * mc);           // Q, K, V codes
  L.scales = at, at += 256;                      // {s, 1/s} of x, Q, K, V, O
  L.part = at, at += round256(part);
  L.tab = at, at += rope_table_bytes(p);
  L.total = at;
  return L;
}

}  // namespace

size_t skiparse_block_workspace_bytes(const skiparse_plan* plan) {
  if (check_plan(plan)) return 0;
  return block_layout(*plan).total;
}

int skiparse_block_fwd_fp8(const skiparse_plan* plan, const void* x, const uint8_t* w_qkvo, const float* dev_w_scales,
                           float rope_theta, const int32_t* rope_dims, void* y, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  if (int e = check_plan(plan)) return e;
  const int d = plan->d;
  if (d != 128) return fail(SKIPARSE_EUNSUPPORTED, "the fp8 block is built for d=128 only (d=%d)", d);
  if (!x || !w_qkvo || !dev_w_scales || !y) return fail(SKIPARSE_EINVAL, "x, w_qkvo, dev_w_scales and y must be non-NULL");
  if (!aligned16(x) || !aligned16(w_qkvo) || !aligned16(y))
    return fail(SKIPARSE_EINVAL, "x, w_qkvo and y must be 16-byte aligned");
  if (((uintptr_t)dev_w_scales & 3u) != 0) return fail(SKIPARSE_EINVAL, "dev_w_scales must be 4-byte aligned");
  RopeGeom r;
  if (int e = rope_setup(*plan, rope_theta, rope_dims, r)) return e;
  const int64_t C = (int64_t)plan->heads * d;
  const int64_t M = (int64_t)plan->B * plan->T * plan->H * plan->W;
  const int64_t mc = M * C;
  if (C > 65536) return fail(SKIPARSE_EUNSUPPORTED, "heads*d = %lld is above 65536", (long long)C);
  if (M >= (int64_t(1) << 31)) return fail(SKIPARSE_EINVAL, "B*T*H*W must stay below 2^31");
  const BlockLayout L = block_layout(*plan);
  if (!workspace || workspace_bytes < L.total)
    return fail(SKIPARSE_EWORKSPACE, "workspace of %zu bytes needed, %zu given", L.total, workspace ? workspace_bytes : 0);
  if (((uintptr_t)workspace & 255u) != 0) return fail(SKIPARSE_EINVAL, "workspace must be 256-byte aligned");
  const size_t wb = (size_t)(4 * C * C);
  if (overlap(y, mc * 2, x, mc * 2) || overlap(y, mc * 2, w_qkvo, wb) || overlap(y, mc * 2, dev_w_scales, 32) ||
      overlap(workspace, L.total, x, mc * 2) ||
      overlap(workspace, L.total, y, mc * 2) || overlap(workspace, L.total, w_qkvo, wb) ||
      overlap(workspace, L.total, dev_w_scales, 32))
    return fail(SKIPARSE_EINVAL, "y and the workspace must not overlap each other or the inputs");

  char* ws = (char*)workspace;
  uint8_t* x8 = (uint8_t*)(ws + L.x8);
  char* b16 = ws + L.qkv16;
  uint8_t* c8 = (uint8_t*)(ws + L.qkv8);
  float* sc = (float*)(ws + L.scales);
  float* part = (float*)(ws + L.part);
  float2* tab = (float2*)(ws + L.tab);

  AttnArgs a;
  int32_t all = 0;
  if (int e = fill_attn_args(plan, 0.f, 0, all, a)) return e;
  a.q = c8;
  a.k = c8 + mc;
  a.v = c8 + 2 * mc;
  a.o = b16;                 // O (bf16) over the Q projection, dead by then
  a.descale = sc + 2;        // {s_q, 1/s_q, s_k, 1/s_k, s_v, 1/s_v}

  (void)hipGetLastError();
  auto hip_fail = [&](hipError_t e, const char* what) {
    return fail(SKIPARSE_EHIP, "%s failed: %s", what, hipGetErrorString(e));
  };
  hipError_t e = launch_quant_fp8(x, 1, mc, x8, sc, kE4M3MaxHost, 1e-12f, part, stream);
  if (e != hipSuccess) return hip_fail(e, "quantization of x");
  for (int i = 0; i < 3; ++i)
    if ((e = launch_gemm_fp8_bf16(x8, w_qkvo + i * C * C, sc + 1, dev_w_scales + 2 * i + 1, b16 + i * mc * 2, M,
                                  (int)C, (int)C, stream)) != hipSuccess)
      return hip_fail(e, "projection");
  if ((e = launch_rope_table(r, rope_theta, tab, stream)) != hipSuccess) return hip_fail(e, "rotary table");
  for (int i = 0; i < 2; ++i)
    if ((e = launch_rope_quant(r, tab, b16 + i * mc * 2, c8 + i * mc, sc + 2 + 2 * i, part, stream)) != hipSuccess)
      return hip_fail(e, "rotary embedding");
  if ((e = launch_quant_fp8(b16 + 2 * mc * 2, 1, mc, c8 + 2 * mc, sc + 6, kE4M3MaxHost, 1e-12f, part, stream)) != hipSuccess)
    return hip_fail(e, "quantization of V");
  if ((e = launch_attn_fp8(a, plan->B, d, stream)) != hipSuccess) return hip_fail(e, "attention");
  if ((e = launch_quant_fp8(b16, 1, mc, x8, sc + 8, kE4M3MaxHost, 1e-12f, part, stream)) != hipSuccess)
    return hip_fail(e, "quantization of O");
  if ((e = launch_gemm_fp8_bf16(x8, w_qkvo + 3 * C * C, sc + 9, dev_w_scales + 7, y, M, (int)C, (int)C, stream)) !=
      hipSuccess)
    return hip_fail(e, "output projection");
  return ok();
}

int skiparse_gemm_fp8(const uint8_t* x, const uint8_t* w, const float* dev_sx, const float* dev_sw, void* y,
                      int64_t M, int32_t N, int32_t K, hipStream_t stream) {
  if (M < 1 || M >= (int64_t(1) << 31)) return fail(SKIPARSE_EINVAL, "M=%lld outside [1, 2^31)", (long long)M);
  if (N < 128 || K < 128 || N % 128 || K % 128 || N > 65536 || K > 65536)
    return fail(SKIPARSE_EUNSUPPORTED, "N=%d and K=%d must be multiples of 128 in [128, 65536]", N, K);
  if (((M + 127) / 128) * (N / 128) >= (int64_t(1) << 31)) return fail(SKIPARSE_EINVAL, "too many tiles");
  if (!x || !w || !dev_sx || !dev_sw || !y) return fail(SKIPARSE_EINVAL, "x, w, dev_sx, dev_sw and y must be non-NULL");
  if (!aligned16(x) || !aligned16(w) || ((uintptr_t)y & 7u) != 0 || ((uintptr_t)dev_sx & 3u) != 0 ||
      ((uintptr_t)dev_sw & 3u) != 0)
    return fail(SKIPARSE_EINVAL, "x and w must be 16-byte aligned, y 8-byte, dev_sx and dev_sw 4-byte");
  const size_t yb = (size_t)M * N * 2;
  if (overlap(y, yb, x, (size_t)M * K) || overlap(y, yb, w, (size_t)N * K) || overlap(y, yb, dev_sx, 4) ||
      overlap(y, yb, dev_sw, 4))
    return fail(SKIPARSE_EINVAL, "y must not overlap the inputs");
  (void)hipGetLastError();
  const hipError_t e = launch_gemm_fp8_bf16(x, w, dev_sx, dev_sw, y, M, N, K, stream);
  if (e != hipSuccess) return fail(SKIPARSE_EHIP, "GEMM launch failed: %s", hipGetErrorString(e));
  return ok();
}

size_t skiparse_rope_fp8_workspace_bytes(const skiparse_plan* plan) {
  if (check_plan(plan)) return 0;
  return rope_table_bytes(*plan) + rope_part_bytes(*plan);
}

int skiparse_rope_fp8(const skiparse_plan* plan, const void* x, float rope_theta, const int32_t* rope_dims,
                      uint8_t* y, float* dev_scale, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (int e = check_plan(plan)) return e;
  RopeGeom r;
  if (int e = rope_setup(*plan, rope_theta, rope_dims, r)) return e;
  if (!x || !y || !dev_scale) return fail(SKIPARSE_EINVAL, "x, y and dev_scale must be non-NULL");
  if (!aligned16(x) || !aligned16(y) || ((uintptr_t)dev_scale & 3u) != 0)
    return fail(SKIPARSE_EINVAL, "x and y must be 16-byte aligned, dev_scale 4-byte aligned");
  const size_t need = rope_table_bytes(*plan) + rope_part_bytes(*plan);
  if (!workspace || workspace_bytes < need)
    return fail(SKIPARSE_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : 0);
  if (((uintptr_t)workspace & 15u) != 0) return fail(SKIPARSE_EINVAL, "workspace must be 16-byte aligned");
  const size_t n = (size_t)r.nvec * 8;
  if (overlap(y, n, x, 2 * n) || overlap(workspace, need, x, 2 * n) || overlap(workspace, need, y, n) ||
      overlap(dev_scale, 8, x, 2 * n) || overlap(dev_scale, 8, y, n) || overlap(dev_scale, 8, workspace, need))
    return fail(SKIPARSE_EINVAL, "x, y, dev_scale and the workspace must not overlap");
  float2* tab = (float2*)workspace;
  float* part = (float*)((char*)workspace + rope_table_bytes(*plan));
  (void)hipGetLastError();
  hipError_t e = launch_rope_table(r, rope_theta, tab, stream);
  if (e == hipSuccess) e = launch_rope_quant(r, tab, x, y, dev_scale, part, stream);
  if (e != hipSuccess) return fail(SKIPARSE_EHIP, "rotary embedding launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
