// C ABI of libhstu (declarations and the layer's definition in include/hstu.h).
// Host side only: argument validation, workspace carve-up and the launch
// sequence  ln_in -> proj -> build_tiles -> attn -> out  on the caller's stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "hstu.h"
#include "kernels.h"

namespace {

thread_local std::string g_err;

hstu_status fail(hstu_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

hstu_status ok() {
  g_err.clear();
  return HSTU_OK;
}

size_t esize(hstu_dtype dt) { return dt == HSTU_BF16 ? 2 : 4; }
size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

hstu_status check_desc(const hstu_desc* d) {
  if (!d) return fail(HSTU_ERR_INVALID_ARG, "desc is NULL");
  if (d->dtype != HSTU_F32 && d->dtype != HSTU_BF16)
    return fail(HSTU_ERR_UNSUPPORTED, "unknown dtype %d", (int)d->dtype);
  if (d->flags & ~(uint32_t)(HSTU_INPUT_NORM | HSTU_RESIDUAL | HSTU_CAND_SHARED_POS | HSTU_VALIDATE |
                             HSTU_REUSE_PLAN | HSTU_SAVED_FWD))
    return fail(HSTU_ERR_INVALID_ARG, "unknown flag bits 0x%x", d->flags);
  if (d->d_model < 32 || d->d_model > 8192 || d->d_model % 32 != 0)
    return fail(HSTU_ERR_UNSUPPORTED, "d_model %d: must be a multiple of 32 in [32, 8192]", d->d_model);
  if (d->num_heads < 1 || d->num_heads > 64)
    return fail(HSTU_ERR_UNSUPPORTED, "num_heads %d: must be in [1, 64]", d->num_heads);
  auto okdim = [](int v) { return v == 32 || v == 64 || v == 128; };
  if (!okdim(d->dqk) || !okdim(d->dv))
    return fail(HSTU_ERR_UNSUPPORTED, "dqk %d / dv %d: each must be 32, 64 or 128", d->dqk, d->dv);
  if (d->dtype == HSTU_F32 && (d->dqk > 64 || d->dv > 64))
    return fail(HSTU_ERR_UNSUPPORTED, "fp32 layers support dqk, dv <= 64");
  if (d->pos_buckets < 1 || d->pos_buckets > 2047 || d->pos_buckets % 2 == 0)
    return fail(HSTU_ERR_INVALID_ARG, "pos_buckets %d: must be odd in [1, 2047]", d->pos_buckets);
  if (d->time_buckets < 1 || d->time_buckets > 2048)
    return fail(HSTU_ERR_INVALID_ARG, "time_buckets %d: must be in [1, 2048]", d->time_buckets);
  if (d->time_sub_bits < 0 || d->time_sub_bits > 4)
    return fail(HSTU_ERR_INVALID_ARG, "time_sub_bits %d: must be in [0, 4]", d->time_sub_bits);
  if (!(d->ln_eps > 0.f) || !std::isfinite(d->ln_eps))
    return fail(HSTU_ERR_INVALID_ARG, "ln_eps must be positive and finite");
  if (d->norm_len < 0) return fail(HSTU_ERR_INVALID_ARG, "norm_len %d < 0", d->norm_len);
  if (d->num_types < 0 || d->num_types > 16)
    return fail(HSTU_ERR_UNSUPPORTED, "num_types %d: must be in [0, 16]", d->num_types);
  return HSTU_OK;
}

hstu_status check_sizes(int64_t T, int32_t B) {
  if (T < 0) return fail(HSTU_ERR_INVALID_ARG, "total_tokens %lld < 0", (long long)T);
  if (T > INT32_MAX - 1024) return fail(HSTU_ERR_UNSUPPORTED, "total_tokens %lld too large", (long long)T);
  if (B < 0) return fail(HSTU_ERR_INVALID_ARG, "batch %d < 0", B);
  if (T > 0 && B == 0) return fail(HSTU_ERR_INVALID_ARG, "total_tokens > 0 with batch 0");
  return HSTU_OK;
}

#define HSTU_REQ(ptr, al, name)                                                         \
  do {                                                                                  \
    if (!(ptr)) return fail(HSTU_ERR_INVALID_ARG, "%s is NULL", name);                  \
    if (!aligned((ptr), (al))) return fail(HSTU_ERR_INVALID_ARG, "%s is not %d-byte aligned", name, (int)(al)); \
  } while (0)

hstu_status check_meta(const int64_t* off, int32_t B, const int64_t* ts, const int32_t* ncand) {
  HSTU_REQ(off, 8, "seq_offsets");
  HSTU_REQ(ts, 8, "timestamps");
  if (ncand && !aligned(ncand, 4)) return fail(HSTU_ERR_INVALID_ARG, "num_candidates is not 4-byte aligned");
  (void)B;
  return HSTU_OK;
}

hstu_status check_tables(const hstu_desc* d, const hstu_bias_tables* t) {
  if (!t) return fail(HSTU_ERR_INVALID_ARG, "tables is NULL");
  HSTU_REQ(t->pos, esize(d->dtype), "tables->pos");
  HSTU_REQ(t->time, esize(d->dtype), "tables->time");
  if (t->pos_head_stride < 0 || t->time_head_stride < 0)
    return fail(HSTU_ERR_INVALID_ARG, "negative table head stride");
  if (t->pos_head_stride != 0 && t->pos_head_stride < d->pos_buckets)
    return fail(HSTU_ERR_INVALID_ARG, "pos_head_stride %d < pos_buckets %d", t->pos_head_stride, d->pos_buckets);
  if (t->time_head_stride != 0 && t->time_head_stride < d->time_buckets)
    return fail(HSTU_ERR_INVALID_ARG, "time_head_stride %d < time_buckets %d", t->time_head_stride, d->time_buckets);
  if (d->num_types > 0) {
    const int nt2 = d->num_types * d->num_types;
    HSTU_REQ(t->type, esize(d->dtype), "tables->type");
    if (t->token_types == nullptr) return fail(HSTU_ERR_INVALID_ARG, "tables->token_types is NULL");
    if (t->type_head_stride < 0 || (t->type_head_stride != 0 && t->type_head_stride < nt2))
      return fail(HSTU_ERR_INVALID_ARG, "type_head_stride %d: must be 0 or >= num_types^2 = %d",
                  t->type_head_stride, nt2);
    if (t->reserved != 0) return fail(HSTU_ERR_INVALID_ARG, "tables->reserved must be 0");
  }
  return HSTU_OK;
}

hstu::AttnTypes layer_types(const hstu_desc* d, const hstu_bias_tables* t) {
  if (d->num_types == 0) return hstu::AttnTypes{nullptr, nullptr, 0};
  return hstu::AttnTypes{t->token_types, t->token_types, d->num_types};
}

hstu_status check_proj_weights(const hstu_desc* d, const hstu_weights* w) {
  if (!w) return fail(HSTU_ERR_INVALID_ARG, "weights is NULL");
  HSTU_REQ(w->w1, 16, "weights->w1");
  HSTU_REQ(w->b1, esize(d->dtype), "weights->b1");
  if (d->flags & HSTU_INPUT_NORM) {
    HSTU_REQ(w->ln_in_g, 16, "weights->ln_in_g");
    HSTU_REQ(w->ln_in_b, 16, "weights->ln_in_b");
  }
  return HSTU_OK;
}

hstu_status check_out_weights(const hstu_desc* d, const hstu_weights* w) {
  if (!w) return fail(HSTU_ERR_INVALID_ARG, "weights is NULL");
  HSTU_REQ(w->w2, 16, "weights->w2");
  HSTU_REQ(w->b2, esize(d->dtype), "weights->b2");
  HSTU_REQ(w->ln_av_g, 16, "weights->ln_av_g");
  HSTU_REQ(w->ln_av_b, 16, "weights->ln_av_b");
  return HSTU_OK;
}

hstu_status check_acts(const hstu_activations* a, bool proj, bool attn) {
  if (!a) return fail(HSTU_ERR_INVALID_ARG, "acts is NULL");
  HSTU_REQ(a->u, 16, "acts->u");
  if (proj || attn) {
    HSTU_REQ(a->v, 16, "acts->v");
    HSTU_REQ(a->q, 16, "acts->q");
    HSTU_REQ(a->k, 16, "acts->k");
  }
  if (!proj) {
    HSTU_REQ(a->av, 16, "acts->av");
    HSTU_REQ(a->av_stats, 8, "acts->av_stats");
  }
  return HSTU_OK;
}

// Workspace carve-up shared by the size query and the layer call.
struct Layout {
  size_t xn, u, v, q, k, av, stats, attn, part, total;
};

// Tk: key rows of the attention pass (T in a layer pass, the cached history
// rows in a candidate pass, which also needs the per-chunk partial AV).
Layout layout(const hstu_desc* d, int64_t T, int32_t B, int64_t Tk, bool cached) {
  const size_t e = esize(d->dtype);
  const size_t H = d->num_heads, hdv = H * d->dv, hdq = H * d->dqk;
  Layout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o += align256(bytes);
    return at;
  };
  L.xn = take((d->flags & HSTU_INPUT_NORM) ? (size_t)T * d->d_model * e : 0);
  L.u = take((size_t)T * hdv * e);
  L.v = take((size_t)T * hdv * e);
  L.q = take((size_t)T * hdq * e);
  L.k = take((size_t)T * hdq * e);
  L.av = take((size_t)T * hdv * e);
  L.stats = take((size_t)T * H * 2 * sizeof(float));
  L.attn = take(hstu::attn_scratch_bytes(T, Tk, B, cached));
  L.part = take(cached ? hstu::cand_partial_bytes(T, d->num_heads, d->dv) : 0);
  L.total = o;
  return L;
}

size_t attn_ws(int64_t T, int32_t B) { return hstu::attn_scratch_bytes(T, B); }

hstu_status device(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(HSTU_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
  return HSTU_OK;
}

hstu_status validate_metadata(const int64_t* off, int32_t B, int64_t T, const int32_t* ncand,
                              hipStream_t s) {
  std::vector<int64_t> h_off((size_t)B + 1);
  std::vector<int32_t> h_nc(ncand ? (size_t)B : 0);
  hstu_status st = device(hipMemcpyAsync(h_off.data(), off, h_off.size() * 8, hipMemcpyDeviceToHost, s),
                          "copy seq_offsets");
  if (st != HSTU_OK) return st;
  if (ncand && B > 0) {
    st = device(hipMemcpyAsync(h_nc.data(), ncand, h_nc.size() * 4, hipMemcpyDeviceToHost, s),
                "copy num_candidates");
    if (st != HSTU_OK) return st;
  }
  st = device(hipStreamSynchronize(s), "synchronise for validation");
  if (st != HSTU_OK) return st;
  if (h_off[0] != 0) return fail(HSTU_ERR_INVALID_ARG, "seq_offsets[0] = %lld, expected 0", (long long)h_off[0]);
  if (h_off[B] != T)
    return fail(HSTU_ERR_INVALID_ARG, "seq_offsets[B] = %lld, expected total_tokens %lld",
                (long long)h_off[B], (long long)T);
  for (int32_t b = 0; b < B; ++b) {
    const int64_t L = h_off[b + 1] - h_off[b];
    if (L < 0) return fail(HSTU_ERR_INVALID_ARG, "seq_offsets decreases at %d", b);
    if (ncand && (h_nc[b] < 0 || h_nc[b] > L))
      return fail(HSTU_ERR_INVALID_ARG, "num_candidates[%d] = %d outside [0, %lld]", b, h_nc[b], (long long)L);
  }
  return HSTU_OK;
}

}  // namespace

extern "C" {

const char* hstu_status_str(hstu_status s) {
  switch (s) {
    case HSTU_OK: return "ok";
    case HSTU_ERR_INVALID_ARG: return "invalid argument";
    case HSTU_ERR_UNSUPPORTED: return "unsupported configuration";
    case HSTU_ERR_WORKSPACE: return "workspace too small";
    case HSTU_ERR_DEVICE: return "device error";
  }
  return "unknown status";
}

const char* hstu_last_error(void) { return g_err.c_str(); }

size_t hstu_workspace_size(const hstu_desc* desc, int64_t T, int32_t B) {
  if (check_desc(desc) != HSTU_OK || check_sizes(T, B) != HSTU_OK) return 0;
  return layout(desc, T, B, T, false).total;
}

size_t hstu_proj_workspace_size(const hstu_desc* desc, int64_t T) {
  if (check_desc(desc) != HSTU_OK || check_sizes(T, 1) != HSTU_OK) return 0;
  if (!(desc->flags & HSTU_INPUT_NORM)) return 0;
  return align256((size_t)T * desc->d_model * esize(desc->dtype));
}

size_t hstu_attn_workspace_size(const hstu_desc* desc, int64_t T, int32_t B) {
  if (check_desc(desc) != HSTU_OK || check_sizes(T, B) != HSTU_OK) return 0;
  return attn_ws(T, B);
}

static hstu_status run_proj(const hstu_desc* d, const void* x, int64_t T, const hstu_weights* w,
                            const hstu_activations* a, void* xn, hipStream_t s, void* pre = nullptr) {
  const void* src = x;
  if (d->flags & HSTU_INPUT_NORM) {
    hstu_status st = device(hstu::launch_ln_in(d->dtype, x, w->ln_in_g, w->ln_in_b, xn, T,
                                               d->d_model, d->ln_eps, s), "ln_in launch");
    if (st != HSTU_OK) return st;
    src = xn;
  }
  return device(hstu::launch_proj(*d, src, T, w->w1, w->b1, a->u, a->v, a->q, a->k, pre, s), "proj launch");
}

static hstu_status run_attn(const hstu_desc* d, const int64_t* off, int32_t B, int64_t T,
                            const int64_t* ts, const int32_t* nc, const hstu_bias_tables* t,
                            const hstu_activations* a, void* scratch, hipStream_t s) {
  const hstu::AttnScratch sc = hstu::attn_scratch(scratch, T, B);
  const hstu::AttnRows rows{off, nc, ts, T, off, ts, T, nullptr, B, false, layer_types(d, t)};
  if (!(d->flags & HSTU_REUSE_PLAN)) {
    const hstu_status st = device(hstu::launch_attn_prep(rows, hstu::kAttnBM, sc, s), "attention prep launch");
    if (st != HSTU_OK) return st;
  }
  return device(hstu::launch_attn(*d, rows, *t, a->q, a->k, a->v, nullptr, nullptr, a->av, a->av_stats, sc, s),
                "attention launch");
}

hstu_status hstu_proj_fwd(const hstu_desc* desc, const void* x, int64_t T, const hstu_weights* w,
                          const hstu_activations* acts, void* ws, size_t ws_bytes,
                          hstu_stream_t stream) {
  hstu_status st;
  if ((st = check_desc(desc)) != HSTU_OK) return st;
  if ((st = check_sizes(T, 1)) != HSTU_OK) return st;
  if (T == 0) return ok();
  HSTU_REQ(x, 16, "x");
  if ((st = check_proj_weights(desc, w)) != HSTU_OK) return st;
  if ((st = check_acts(acts, true, false)) != HSTU_OK) return st;
  const size_t need = hstu_proj_workspace_size(desc, T);
  if (need > 0 && (!ws || ws_bytes < need || !aligned(ws, 256)))
    return fail(HSTU_ERR_WORKSPACE, "workspace: need %zu bytes (256-aligned), got %zu", need, ws_bytes);
  if ((st = run_proj(desc, x, T, w, acts, ws, (hipStream_t)stream)) != HSTU_OK) return st;
  return ok();
}

hstu_status hstu_attn_fwd(const hstu_desc* desc, const int64_t* off, int32_t B, int64_t T,
                          const int64_t* ts, const int32_t* nc, const hstu_bias_tables* tables,
                          const hstu_activations* acts, void* ws, size_t ws_bytes,
                          hstu_stream_t stream) {
  hstu_status st;
  if ((st = check_desc(desc)) != HSTU_OK) return st;
  if ((st = check_sizes(T, B)) != HSTU_OK) return st;
  if (T == 0) return ok();
  if ((st = check_meta(off, B, ts, nc)) != HSTU_OK) return st;
  if ((st = check_tables(desc, tables)) != HSTU_OK) return st;
  if ((st = check_acts(acts, false, true)) != HSTU_OK) return st;
  const size_t need = attn_ws(T, B);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(HSTU_ERR_WORKSPACE, "workspace: need %zu bytes (256-aligned), got %zu", need, ws_bytes);
  hipStream_t s = (hipStream_t)stream;
  if (desc->flags & HSTU_VALIDATE)
    if ((st = validate_metadata(off, B, T, nc, s)) != HSTU_OK) return st;
  if ((st = run_attn(desc, off, B, T, ts, nc, tables, acts, ws, s)) != HSTU_OK) return st;
  return ok();
}

hstu_status hstu_gate_fwd(const hstu_desc* desc, int64_t T, const hstu_weights* w,
                          const hstu_activations* acts, void* z, hstu_stream_t stream) {
  hstu_status st;
  if ((st = check_desc(desc)) != HSTU_OK) return st;
  if ((st = check_sizes(T, 1)) != HSTU_OK) return st;
  if (T == 0) return ok();
  HSTU_REQ(z, 16, "z");
  if ((st = check_out_weights(desc, w)) != HSTU_OK) return st;
  if ((st = check_acts(acts, false, false)) != HSTU_OK) return st;
  st = device(hstu::launch_gate(*desc, T, *w, acts->u, acts->av, acts->av_stats, z, (hipStream_t)stream),
              "gate launch");
  if (st != HSTU_OK) return st;
  return ok();
}

hstu_status hstu_out_fwd(const hstu_desc* desc, const void* x, int64_t T, const hstu_weights* w,
                         const hstu_activations* acts, void* out, void* z, hstu_stream_t stream) {
  hstu_status st;
  if ((st = check_desc(desc)) != HSTU_OK) return st;
  if ((st = check_sizes(T, 1)) != HSTU_OK) return st;
  if (T == 0) return ok();
  if (desc->flags & HSTU_RESIDUAL) HSTU_REQ(x, 16, "x");
  HSTU_REQ(out, 16, "out");
  HSTU_REQ(z, 16, "z");
  if ((st = check_out_weights(desc, w)) != HSTU_OK) return st;
  if ((st = check_acts(acts, false, false)) != HSTU_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if ((st = device(hstu::launch_gate(*desc, T, *w, acts->u, acts->av, acts->av_stats, z, s), "gate launch")) !=
      HSTU_OK)
    return st;
  if ((st = device(hstu::launch_f2(*desc, x, T, *w, z, out, s), "f2 launch")) != HSTU_OK) return st;
  return ok();
}

// Host-side checks of hstu_layer_fwd's arguments (no device access).
static hstu_status check_layer_args(const hstu_desc* desc, const void* x, const int64_t* off, int32_t B, int64_t T,
                                    const int64_t* ts, const int32_t* nc, const hstu_weights* w,
                                    const hstu_bias_tables* tables, const void* out) {
  hstu_status st;
  if ((st = check_desc(desc)) != HSTU_OK) return st;
  if ((st = check_sizes(T, B)) != HSTU_OK) return st;
  if (T == 0) return HSTU_OK;
  HSTU_REQ(x, 16, "x");
  HSTU_REQ(out, 16, "out");
  if ((st = check_meta(off, B, ts, nc)) != HSTU_OK) return st;
  if ((st = check_proj_weights(desc, w)) != HSTU_OK) return st;
  if ((st = check_out_weights(desc, w)) != HSTU_OK) return st;
  return check_tables(desc, tables);
}

hstu_status hstu_layer_fwd(const hstu_desc* desc, const void* x, const int64_t* off, int32_t B,
                           int64_t T, const int64_t* ts, const int32_t* nc, const hstu_weights* w,
                           const hstu_bias_tables* tables, void* out, void* ws, size_t ws_bytes,
                           hstu_stream_t stream) {
  hstu_status st;
  if ((st = check_layer_args(desc, x, off, B, T, ts, nc, w, tables, out)) != HSTU_OK) return st;
  if (T == 0) return ok();
  const Layout L = layout(desc, T, B, T, false);
  if (!ws || ws_bytes < L.total || !aligned(ws, 256))
    return fail(HSTU_ERR_WORKSPACE, "workspace: need %zu bytes (256-aligned), got %zu", L.total, ws_bytes);
  hipStream_t s = (hipStream_t)stream;
  if (desc->flags & HSTU_VALIDATE)
    if ((st = validate_metadata(off, B, T, nc, s)) != HSTU_OK) return st;
  char* base = (char*)ws;
  hstu_activations a;
  a.u = base + L.u;
  a.v = base + L.v;
  a.q = base + L.q;
  a.k = base + L.k;
  a.av = base + L.av;
  a.av_stats = (float*)(base + L.stats);
  if ((st = run_proj(desc, x, T, w, &a, base + L.xn, s)) != HSTU_OK) return st;
  if ((st = run_attn(desc, off, B, T, ts, nc, tables, &a, base + L.attn, s)) != HSTU_OK)
    return st;
  // Z takes the V region: V [H, T, dv] has Z's size and is dead after stage 2.
  void* z = base + L.v;
  if ((st = device(hstu::launch_gate(*desc, T, *w, a.u, a.av, a.av_stats, z, s), "gate launch")) != HSTU_OK)
    return st;
  if ((st = device(hstu::launch_f2(*desc, x, T, *w, z, out, s), "f2 launch")) != HSTU_OK) return st;
  return ok();
}

// The no-allocation entry point's scratch: one array per GPU (each device
// holds its own copy of a __device__ variable), looked up once per device.
// In host code `scratch` names a host-side stand-in, never the device memory:
// only the addresses from hipGetSymbolAddress are passed to kernels.
static __device__ __align__(256) unsigned char scratch[HSTU_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

static hstu_status device_scratch(void** ptr) {
  int dev = -1;
  hstu_status st = device(hipGetDevice(&dev), "hipGetDevice");
  if (st != HSTU_OK) return st;
  if (dev < 0 || dev >= kMaxDevices) return fail(HSTU_ERR_UNSUPPORTED, "device %d >= %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if ((st = device(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)")) != HSTU_OK)
      return st;
    if (!p || !aligned(p, 256)) return fail(HSTU_ERR_DEVICE, "scratch array address %p not 256-aligned", p);
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return HSTU_OK;
}

hstu_status hstu_layer_fwd_noalloc(const hstu_desc* desc, const void* x, const int64_t* off, int32_t B,
                                   int64_t T, const int64_t* ts, const int32_t* nc, const hstu_weights* w,
                                   const hstu_bias_tables* tables, void* out, hstu_stream_t stream) {
  hstu_status st;
  if ((st = check_layer_args(desc, x, off, B, T, ts, nc, w, tables, out)) != HSTU_OK) return st;
  if (desc->flags & HSTU_VALIDATE)
    return fail(HSTU_ERR_INVALID_ARG, "HSTU_VALIDATE copies to the host and synchronises: not available here");
  if (T == 0) return ok();
  const size_t need = layout(desc, T, B, T, false).total;
  if (need > HSTU_NOALLOC_SCRATCH_BYTES)
    return fail(HSTU_ERR_WORKSPACE, "%lld tokens in %d sequences need %zu bytes of scratch; the limit is %zu",
                (long long)T, B, need, (size_t)HSTU_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if ((st = device_scratch(&ws)) != HSTU_OK) return st;
  return hstu_layer_fwd(desc, x, off, B, T, ts, nc, w, tables, out, ws, HSTU_NOALLOC_SCRATCH_BYTES, stream);
}

size_t hstu_cand_workspace_size(const hstu_desc* desc, int64_t Tc, int64_t Th, int32_t B) {
  if (check_desc(desc) != HSTU_OK || check_sizes(Tc, B) != HSTU_OK || check_sizes(Th, B) != HSTU_OK) return 0;
  return layout(desc, Tc, B, Th, true).total;
}

hstu_status hstu_cand_fwd(const hstu_desc* desc, const void* x, const int64_t* coff, int32_t B, int64_t Tc,
                          const int64_t* cts, const int32_t* mtotal, const int64_t* hoff, int64_t Th,
                          const int64_t* hts, const void* hk, const void* hv, const hstu_weights* w,
                          const hstu_bias_tables* tables, void* out, void* ws, size_t ws_bytes,
                          hstu_stream_t stream) {
  hstu_status st;
  if ((st = check_desc(desc)) != HSTU_OK) return st;
  if (!(desc->flags & HSTU_CAND_SHARED_POS))
    return fail(HSTU_ERR_UNSUPPORTED, "the candidate pass needs HSTU_CAND_SHARED_POS");
  if ((st = check_sizes(Tc, B)) != HSTU_OK) return st;
  if ((st = check_sizes(Th, B)) != HSTU_OK) return st;
  if (Tc == 0) return ok();
  HSTU_REQ(x, 16, "x");
  HSTU_REQ(out, 16, "out");
  HSTU_REQ(mtotal, 4, "num_candidates");
  if ((st = check_meta(coff, B, cts, nullptr)) != HSTU_OK) return st;
  HSTU_REQ(hoff, 8, "hist_offsets");
  if (Th > 0) {  // with no history rows the cache may be empty (NULL)
    HSTU_REQ(hk, 16, "hist_k");
    HSTU_REQ(hv, 16, "hist_v");
    HSTU_REQ(hts, 8, "hist_ts");
    if (desc->num_types > 0 && tables && !tables->hist_types)
      return fail(HSTU_ERR_INVALID_ARG, "tables->hist_types is NULL");
  }
  if ((st = check_proj_weights(desc, w)) != HSTU_OK) return st;
  if ((st = check_out_weights(desc, w)) != HSTU_OK) return st;
  if ((st = check_tables(desc, tables)) != HSTU_OK) return st;
  const Layout L = layout(desc, Tc, B, Th, true);
  if (!ws || ws_bytes < L.total || !aligned(ws, 256))
    return fail(HSTU_ERR_WORKSPACE, "workspace: need %zu bytes (256-aligned), got %zu", L.total, ws_bytes);
  hipStream_t s = (hipStream_t)stream;
  if (desc->flags & HSTU_VALIDATE) {
    if ((st = validate_metadata(coff, B, Tc, nullptr, s)) != HSTU_OK) return st;
    if ((st = validate_metadata(hoff, B, Th, nullptr, s)) != HSTU_OK) return st;
  }
  char* base = (char*)ws;
  hstu_activations a;
  a.u = base + L.u;
  a.v = base + L.v;
  a.q = base + L.q;
  a.k = base + L.k;
  a.av = base + L.av;
  a.av_stats = (float*)(base + L.stats);
  if ((st = run_proj(desc, x, Tc, w, &a, base + L.xn, s)) != HSTU_OK) return st;
  const hstu::AttnScratch sc = hstu::attn_scratch(base + L.attn, Tc, Th, B, true);
  const hstu::AttnTypes types = desc->num_types > 0
                                    ? hstu::AttnTypes{tables->token_types, tables->hist_types, desc->num_types}
                                    : hstu::AttnTypes{nullptr, nullptr, 0};
  const hstu::AttnRows rows{coff, nullptr, cts, Tc, hoff, hts, Th, mtotal, B, true, types};
  if (!(desc->flags & HSTU_REUSE_PLAN))
    if ((st = device(hstu::launch_attn_prep(rows, hstu::kAttnBM, sc, s), "attention prep launch")) != HSTU_OK)
      return st;
  float* part = (float*)(base + L.part);
  if ((st = device(hstu::launch_attn_cached(*desc, rows, *tables, a.q, hk, hv, a.k, a.v, part, sc, s),
                   "attention launch")) != HSTU_OK)
    return st;
  // Z takes the V region, dead once the attention (self terms included) has run.
  void* z = base + L.v;
  if ((st = device(hstu::launch_cand_gate(*desc, coff, B, Tc, sc.nsplit, part, *w, a.u, z, s), "gate launch")) !=
      HSTU_OK)
    return st;
  if ((st = device(hstu::launch_f2(*desc, x, Tc, *w, z, out, s), "f2 launch")) != HSTU_OK) return st;
  return ok();
}

// Backward workspace: the forward's buffers, then the backward's.
struct BwdLayout {
  Layout f;
  size_t pre, z, dz, dav, gterm_av, bterm_av, tab_part, dpre_t, w2t, dyt, zt, w1t, dpret, xnt, dxn, gterm_in,
      ctmp, wsplit, total;
  int64_t Tp;
};

static BwdLayout bwd_layout(const hstu_desc* d, int64_t T, int32_t B) {
  BwdLayout L{};
  L.f = layout(d, T, B, T, false);
  const size_t e = esize(d->dtype);
  const int64_t K2 = (int64_t)d->num_heads * d->dv, N1 = 2 * (int64_t)d->num_heads * (d->dqk + d->dv);
  const int64_t dm = d->d_model;
  L.Tp = (T + 63) / 64 * 64;
  size_t o = L.f.total;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o += align256(bytes);
    return at;
  };
  L.pre = take((size_t)T * N1 * e);
  L.z = take((size_t)T * K2 * e);
  L.dz = take((size_t)T * K2 * 4);
  L.dav = take((size_t)T * K2 * e);
  const int64_t rchunks = (T + 31) / 32;  // the LayerNorm backward kernels' 32-row partial sums
  L.gterm_av = take((size_t)rchunks * K2 * 4);
  L.bterm_av = take((size_t)rchunks * K2 * 4);
  L.tab_part = take((size_t)hstu::attn_max_tiles(T, B) * d->num_heads * (d->pos_buckets + d->time_buckets) * 4);
  L.dpre_t = take((size_t)T * N1 * e);
  L.w2t = take((size_t)K2 * dm * e);
  // transposed copies for the weight gradients: fp32 layers only (bf16 layers
  // read the token-major operands directly)
  const bool tcopies = d->dtype != HSTU_BF16;
  L.dyt = take(tcopies ? (size_t)dm * L.Tp * e : 0);
  L.zt = take(tcopies ? (size_t)K2 * L.Tp * e : 0);
  L.w1t = take((size_t)dm * N1 * e);
  L.dpret = take(tcopies ? (size_t)N1 * L.Tp * e : 0);
  L.xnt = take(tcopies ? (size_t)dm * L.Tp * e : 0);
  L.dxn = take((size_t)T * dm * 4);
  L.gterm_in = take((size_t)2 * rchunks * dm * 4);
  const int64_t cmax = N1 > dm ? (N1 > K2 ? N1 : K2) : (dm > K2 ? dm : K2);
  L.ctmp = take(hstu::colsum_tmp_bytes(T, cmax));
  L.wsplit = take((size_t)hstu::kGemmMaxSplit * (size_t)(N1 > K2 ? N1 : K2) * dm * 4);
  L.total = o;
  return L;
}

static hstu_status check_bwd_desc(const hstu_desc* d) {
  hstu_status st;
  if ((st = check_desc(d)) != HSTU_OK) return st;
  if (d->num_types != 0) return fail(HSTU_ERR_UNSUPPORTED, "the backward pass has no token-type term yet");
  if (d->dqk != d->dv) return fail(HSTU_ERR_UNSUPPORTED, "the backward pass needs dqk == dv");
  if (d->pos_buckets + d->time_buckets > 2048)
    return fail(HSTU_ERR_UNSUPPORTED, "the backward pass needs pos_buckets + time_buckets <= 2048");
  if (d->d_model > 2048 || d->num_heads * d->dv > 2048)
    return fail(HSTU_ERR_UNSUPPORTED, "the backward pass needs d_model <= 2048 and num_heads * dv <= 2048");
  return HSTU_OK;
}

size_t hstu_bwd_workspace_size(const hstu_desc* desc, int64_t T, int32_t B) {
  if (check_bwd_desc(desc) != HSTU_OK || check_sizes(T, B) != HSTU_OK) return 0;
  return bwd_layout(desc, T, B).total;
}

// The forward into a backward workspace: U, V, Q, K and the pre-activation
// x~ W1^T + b1; AV and its statistics (and the work list); Z in its own
// region (V stays); then f2 into out when out is given.
static hstu_status fwd_into_bwd_layout(const hstu_desc* desc, const void* x, const int64_t* off, int32_t B,
                                       int64_t T, const int64_t* ts, const int32_t* nc, const hstu_weights* w,
                                       const hstu_bias_tables* tables, const BwdLayout& L, char* base, void* out,
                                       hipStream_t s) {
  hstu_status st;
  hstu_activations a;
  a.u = base + L.f.u;
  a.v = base + L.f.v;
  a.q = base + L.f.q;
  a.k = base + L.f.k;
  a.av = base + L.f.av;
  a.av_stats = (float*)(base + L.f.stats);
  if ((st = run_proj(desc, x, T, w, &a, base + L.f.xn, s, base + L.pre)) != HSTU_OK) return st;
  if ((st = run_attn(desc, off, B, T, ts, nc, tables, &a, base + L.f.attn, s)) != HSTU_OK) return st;
  void* z = base + L.z;
  if ((st = device(hstu::launch_gate(*desc, T, *w, a.u, a.av, a.av_stats, z, s), "gate launch")) != HSTU_OK) return st;
  if (out)
    if ((st = device(hstu::launch_f2(*desc, x, T, *w, z, out, s), "f2 launch")) != HSTU_OK) return st;
  return HSTU_OK;
}

hstu_status hstu_layer_fwd_train(const hstu_desc* desc, const void* x, const int64_t* off, int32_t B, int64_t T,
                                 const int64_t* ts, const int32_t* nc, const hstu_weights* w,
                                 const hstu_bias_tables* tables, void* out, void* ws, size_t ws_bytes,
                                 hstu_stream_t stream) {
  hstu_status st;
  if ((st = check_bwd_desc(desc)) != HSTU_OK) return st;
  if ((st = check_sizes(T, B)) != HSTU_OK) return st;
  if (T == 0) return ok();
  HSTU_REQ(x, 16, "x");
  HSTU_REQ(out, 16, "out");
  if ((st = check_meta(off, B, ts, nc)) != HSTU_OK) return st;
  if ((st = check_proj_weights(desc, w)) != HSTU_OK) return st;
  if ((st = check_out_weights(desc, w)) != HSTU_OK) return st;
  if ((st = check_tables(desc, tables)) != HSTU_OK) return st;
  const BwdLayout L = bwd_layout(desc, T, B);
  if (!ws || ws_bytes < L.total || !aligned(ws, 256))
    return fail(HSTU_ERR_WORKSPACE, "workspace: need %zu bytes (256-aligned), got %zu", L.total, ws_bytes);
  hipStream_t s = (hipStream_t)stream;
  if (desc->flags & HSTU_VALIDATE)
    if ((st = validate_metadata(off, B, T, nc, s)) != HSTU_OK) return st;
  if ((st = fwd_into_bwd_layout(desc, x, off, B, T, ts, nc, w, tables, L, (char*)ws, out, s)) != HSTU_OK) return st;
  return ok();
}

hstu_status hstu_layer_bwd(const hstu_desc* desc, const void* x, const int64_t* off, int32_t B, int64_t T,
                           const int64_t* ts, const int32_t* nc, const hstu_weights* w,
                           const hstu_bias_tables* tables, const void* dy, void* dx, const hstu_grads* g,
                           void* ws, size_t ws_bytes, hstu_stream_t stream) {
  hstu_status st;
  if ((st = check_bwd_desc(desc)) != HSTU_OK) return st;
  if ((st = check_sizes(T, B)) != HSTU_OK) return st;
  if (!g) return fail(HSTU_ERR_INVALID_ARG, "grads is NULL");
  const float* gp[] = {g->w1, g->b1, g->w2, g->b2, g->ln_in_g, g->ln_in_b, g->ln_av_g, g->ln_av_b, g->pos, g->time};
  for (const float* p : gp)
    if (!p || !aligned(p, 4)) return fail(HSTU_ERR_INVALID_ARG, "a gradient pointer is NULL or misaligned");
  HSTU_REQ(x, 16, "x");
  HSTU_REQ(dy, 16, "dy");
  HSTU_REQ(dx, 16, "dx");
  if ((st = check_meta(off, B, ts, nc)) != HSTU_OK) return st;
  if ((st = check_proj_weights(desc, w)) != HSTU_OK) return st;
  if ((st = check_out_weights(desc, w)) != HSTU_OK) return st;
  if ((st = check_tables(desc, tables)) != HSTU_OK) return st;
  const BwdLayout L = bwd_layout(desc, T, B);
  if (!ws || ws_bytes < L.total || !aligned(ws, 256))
    return fail(HSTU_ERR_WORKSPACE, "workspace: need %zu bytes (256-aligned), got %zu", L.total, ws_bytes);
  hipStream_t s = (hipStream_t)stream;
  if (desc->flags & HSTU_VALIDATE)
    if ((st = validate_metadata(off, B, T, nc, s)) != HSTU_OK) return st;
  const hstu_dtype dt = desc->dtype;
  const int64_t K2 = (int64_t)desc->num_heads * desc->dv, N1 = 2 * (int64_t)desc->num_heads * (desc->dqk + desc->dv);
  const int dm = desc->d_model;
  char* base = (char*)ws;
  auto F = [&](size_t o) { return (float*)(base + o); };
  float* ctmp = F(L.ctmp);
  auto colsum = [&](bool f32, const void* src, int64_t R, int64_t C, float* dst) {
    return device(hstu::launch_colsum(dt, f32, src, R, C, ctmp, dst, s), "column-sum launch");
  };
  if (T == 0) {  // no tokens: every gradient is zero
    if ((st = colsum(true, ctmp, 0, N1 * dm, g->w1)) != HSTU_OK) return st;
    const std::pair<float*, int64_t> z[] = {{g->b1, N1}, {g->w2, dm * K2}, {g->b2, dm}, {g->ln_in_g, dm},
                                            {g->ln_in_b, dm}, {g->ln_av_g, K2}, {g->ln_av_b, K2},
                                            {g->pos, (int64_t)desc->num_heads * desc->pos_buckets},
                                            {g->time, (int64_t)desc->num_heads * desc->time_buckets}};
    for (const auto& p : z)
      if ((st = colsum(true, ctmp, 0, p.second, p.first)) != HSTU_OK) return st;
    return ok();
  }
  hstu_activations a;
  a.u = base + L.f.u;
  a.v = base + L.f.v;
  a.q = base + L.f.q;
  a.k = base + L.f.k;
  a.av = base + L.f.av;
  a.av_stats = F(L.f.stats);
  const bool norm = (desc->flags & HSTU_INPUT_NORM) != 0;
  const void* xn = norm ? (const void*)(base + L.f.xn) : x;
  void* z = base + L.z;
  if (!(desc->flags & HSTU_SAVED_FWD))
    if ((st = fwd_into_bwd_layout(desc, x, off, B, T, ts, nc, w, tables, L, base, nullptr, s)) != HSTU_OK) return st;
  // f2: dZ = dY W2, dW2 = dY^T Z, db2 = sum dY
  if ((st = device(hstu::launch_transpose(dt, w->w2, dm, K2, dm, base + L.w2t, s), "transpose")) != HSTU_OK) return st;
  if ((st = device(hstu::launch_gemm_nt_f32(dt, dy, base + L.w2t, F(L.dz), T, (int)K2, dm, nullptr, s), "gemm")) != HSTU_OK)
    return st;
  const int64_t split_cap = (int64_t)hstu::kGemmMaxSplit * (N1 > K2 ? N1 : K2) * dm;  // L.wsplit, floats
  if (dt == HSTU_BF16) {
    if ((st = device(hstu::launch_gemm_tn_f32(dy, z, g->w2, dm, (int)K2, T, F(L.wsplit), split_cap, s), "gemm")) !=
        HSTU_OK)
      return st;
  } else {
    if ((st = device(hstu::launch_transpose(dt, dy, T, dm, L.Tp, base + L.dyt, s), "transpose")) != HSTU_OK) return st;
    if ((st = device(hstu::launch_transpose(dt, z, T, K2, L.Tp, base + L.zt, s), "transpose")) != HSTU_OK) return st;
    if ((st = device(hstu::launch_gemm_nt_f32(dt, base + L.dyt, base + L.zt, g->w2, dm, (int)K2, (int)L.Tp,
                                              F(L.wsplit), s),
                     "gemm")) != HSTU_OK)
      return st;
  }
  if ((st = colsum(false, dy, T, dm, g->b2)) != HSTU_OK) return st;
  // Each of dU, dV, dQ, dK goes out as its pre-activation gradient:
  // dpre = d(u|v|q|k) * SiLU'(x~ W1^T + b1), from the saved pre-activation.
  // Gate and LayerNorm over the merged heads (dU, dL/dAV):
  void* dpre = base + L.dpre_t;
  if ((st = device(hstu::launch_gate_bwd(*desc, T, *w, F(L.dz), a.u, a.av, a.av_stats, base + L.pre, dpre,
                                         base + L.dav, F(L.gterm_av), F(L.bterm_av), g->ln_av_g, g->ln_av_b, s),
                   "gate backward launch")) != HSTU_OK)
    return st;
  // attention: dV, dQ, dK; the bias tables
  const hstu::AttnScratch sc = hstu::attn_scratch(base + L.f.attn, T, B);
  if ((st = device(hstu::launch_attn_bwd(*desc, off, nc, B, T, ts, *tables, a.q, a.k, a.v, base + L.dav, nullptr,
                                         base + L.pre, dpre, F(L.tab_part), g->pos, g->time, sc, s),
                   "attention backward launch")) != HSTU_OK)
    return st;
  // f1: db1 = column sums of dpre, dW1 = dpre^T x~, dx~ = dpre W1
  if ((st = colsum(false, dpre, T, N1, g->b1)) != HSTU_OK) return st;
  if ((st = device(hstu::launch_transpose(dt, w->w1, N1, dm, N1, base + L.w1t, s), "transpose")) != HSTU_OK) return st;
  if ((st = device(hstu::launch_gemm_nt_f32(dt, base + L.dpre_t, base + L.w1t, F(L.dxn), T, dm, (int)N1, nullptr, s), "gemm")) !=
      HSTU_OK)
    return st;
  if (dt == HSTU_BF16) {
    if ((st = device(hstu::launch_gemm_tn_f32(base + L.dpre_t, xn, g->w1, (int)N1, dm, T, F(L.wsplit), split_cap, s),
                     "gemm")) != HSTU_OK)
      return st;
  } else {
    if ((st = device(hstu::launch_transpose(dt, base + L.dpre_t, T, N1, L.Tp, base + L.dpret, s), "transpose")) !=
        HSTU_OK)
      return st;
    if ((st = device(hstu::launch_transpose(dt, xn, T, dm, L.Tp, base + L.xnt, s), "transpose")) != HSTU_OK) return st;
    if ((st = device(hstu::launch_gemm_nt_f32(dt, base + L.dpret, base + L.xnt, g->w1, N1, dm, (int)L.Tp,
                                              F(L.wsplit), s),
                     "gemm")) != HSTU_OK)
      return st;
  }
  // input LayerNorm and the residual
  // the two sets of partial rows (ceil(T / 32) x d_model each) share one region
  float* gp_in = F(L.gterm_in);
  float* bp_in = gp_in + ((T + 31) / 32) * (int64_t)dm;
  if ((st = device(hstu::launch_ln_bwd(*desc, x, F(L.dxn), *w, dy, T, dx, gp_in, bp_in, g->ln_in_g, g->ln_in_b, s),
                   "ln backward launch")) != HSTU_OK)
    return st;
  return ok();
}

static size_t attn_bwd_ws(const hstu_desc* d, int64_t T, int32_t B, size_t* part_off) {
  const size_t a = align256(hstu::attn_scratch_bytes(T, B));
  if (part_off) *part_off = a;
  return a + align256((size_t)hstu::attn_max_tiles(T, B) * d->num_heads * (d->pos_buckets + d->time_buckets) * 4);
}

size_t hstu_attn_bwd_workspace_size(const hstu_desc* desc, int64_t T, int32_t B) {
  if (check_bwd_desc(desc) != HSTU_OK || check_sizes(T, B) != HSTU_OK) return 0;
  return attn_bwd_ws(desc, T, B, nullptr);
}

hstu_status hstu_attn_bwd(const hstu_desc* desc, const int64_t* off, int32_t B, int64_t T, const int64_t* ts,
                          const int32_t* nc, const hstu_bias_tables* tables, const hstu_activations* acts,
                          const void* dav, float* dqkv, float* dpos, float* dtime, void* ws, size_t ws_bytes,
                          hstu_stream_t stream) {
  hstu_status st;
  if ((st = check_bwd_desc(desc)) != HSTU_OK) return st;
  if ((st = check_sizes(T, B)) != HSTU_OK) return st;
  if (T == 0) return ok();
  if ((st = check_meta(off, B, ts, nc)) != HSTU_OK) return st;
  if ((st = check_tables(desc, tables)) != HSTU_OK) return st;
  if (!acts) return fail(HSTU_ERR_INVALID_ARG, "acts is NULL");
  HSTU_REQ(acts->q, 16, "acts->q");
  HSTU_REQ(acts->k, 16, "acts->k");
  HSTU_REQ(acts->v, 16, "acts->v");
  HSTU_REQ(dav, 16, "dav");
  HSTU_REQ(dqkv, 16, "dqkv");
  HSTU_REQ(dpos, 4, "dpos");
  HSTU_REQ(dtime, 4, "dtime");
  size_t part_off = 0;
  const size_t need = attn_bwd_ws(desc, T, B, &part_off);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(HSTU_ERR_WORKSPACE, "workspace: need %zu bytes (256-aligned), got %zu", need, ws_bytes);
  hipStream_t s = (hipStream_t)stream;
  if (desc->flags & HSTU_VALIDATE)
    if ((st = validate_metadata(off, B, T, nc, s)) != HSTU_OK) return st;
  const hstu::AttnScratch sc = hstu::attn_scratch(ws, T, B);
  if (!(desc->flags & HSTU_REUSE_PLAN)) {
    const hstu::AttnRows rows{off, nc, ts, T, off, ts, T, nullptr, B, false, layer_types(desc, tables)};
    if ((st = device(hstu::launch_attn_prep(rows, hstu::kAttnBM, sc, s), "attention prep launch")) != HSTU_OK)
      return st;
  }
  return device(hstu::launch_attn_bwd(*desc, off, nc, B, T, ts, *tables, acts->q, acts->k, acts->v, dav, dqkv,
                                      nullptr, nullptr, (float*)((char*)ws + part_off), dpos, dtime, sc, s),
                "attention backward launch");
}

size_t hstu_sl_workspace_size(int32_t B) { return B < 0 ? 0 : align256(((size_t)B + 1) * sizeof(int32_t)); }

hstu_status hstu_sl_sample(const int64_t* off, int32_t B, int64_t T, int32_t max_len, float alpha, const float* u,
                           const uint32_t* keys, int64_t* out_off, int64_t* out_rows, void* ws, size_t ws_bytes,
                           hstu_stream_t stream) {
  hstu_status st;
  if ((st = check_sizes(T, B)) != HSTU_OK) return st;
  if (max_len < 1) return fail(HSTU_ERR_INVALID_ARG, "max_len %d < 1", max_len);
  if (!(alpha > 0.f && alpha <= 2.f)) return fail(HSTU_ERR_INVALID_ARG, "alpha %g: must be in (0, 2]", (double)alpha);
  HSTU_REQ(off, 8, "seq_offsets");
  HSTU_REQ(out_off, 8, "out_offsets");
  if (B > 0) HSTU_REQ(u, 4, "u");
  if (T > 0) {
    HSTU_REQ(keys, 4, "keys");
    HSTU_REQ(out_rows, 8, "out_rows");
  }
  const size_t need = hstu_sl_workspace_size(B);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(HSTU_ERR_WORKSPACE, "workspace: need %zu bytes (256-aligned), got %zu", need, ws_bytes);
  // thresholds in float64, as C pow gives them: N^(alpha/2), its floor, N^alpha
  const double thr = std::pow((double)max_len, (double)alpha / 2.0);
  const int64_t k = (int64_t)std::floor(thr);
  const double na = std::pow((double)max_len, (double)alpha);
  return device(hstu::launch_sl_sample(off, B, T, u, keys, thr, k, na, out_off, out_rows, (int32_t*)ws,
                                       (hipStream_t)stream),
                "stochastic-length launch");
}

hstu_status hstu_gather_rows(const void* src, int64_t src_rows, int64_t row_bytes, const int64_t* rows,
                             const int64_t* num_rows, int64_t max_rows, void* dst, hstu_stream_t stream) {
  if (src_rows < 0 || row_bytes < 0 || max_rows < 0)
    return fail(HSTU_ERR_INVALID_ARG, "negative size (src_rows %lld, row_bytes %lld, max_rows %lld)",
                (long long)src_rows, (long long)row_bytes, (long long)max_rows);
  if (max_rows == 0 || row_bytes == 0) return ok();
  if (src_rows == 0) return fail(HSTU_ERR_INVALID_ARG, "rows to gather from an empty source");
  if (!src || !dst) return fail(HSTU_ERR_INVALID_ARG, "src or dst is NULL");
  HSTU_REQ(rows, 8, "rows");
  HSTU_REQ(num_rows, 8, "num_rows");
  return device(hstu::launch_gather_rows(src, src_rows, row_bytes, rows, num_rows, max_rows, dst,
                                         (hipStream_t)stream),
                "gather launch");
}

hstu_status hstu_debug_indices(const hstu_desc* desc, const int64_t* off, int32_t B, int64_t T,
                               const int64_t* ts, const int32_t* nc, const int64_t* pairs,
                               int64_t n, int64_t* out, hstu_stream_t stream) {
  hstu_status st;
  if ((st = check_desc(desc)) != HSTU_OK) return st;
  if ((st = check_sizes(T, B)) != HSTU_OK) return st;
  if (n < 0) return fail(HSTU_ERR_INVALID_ARG, "n_pairs %lld < 0", (long long)n);
  if (n == 0) return ok();
  if ((st = check_meta(off, B, ts, nc)) != HSTU_OK) return st;
  HSTU_REQ(pairs, 8, "pairs");
  HSTU_REQ(out, 8, "out");
  hipStream_t s = (hipStream_t)stream;
  if (desc->flags & HSTU_VALIDATE) {
    if ((st = validate_metadata(off, B, T, nc, s)) != HSTU_OK) return st;
    std::vector<int64_t> hp((size_t)n * 2);
    if ((st = device(hipMemcpyAsync(hp.data(), pairs, hp.size() * 8, hipMemcpyDeviceToHost, s),
                     "copy pairs")) != HSTU_OK)
      return st;
    if ((st = device(hipStreamSynchronize(s), "synchronise")) != HSTU_OK) return st;
    for (size_t i = 0; i < hp.size(); ++i)
      if (hp[i] < 0 || hp[i] >= T) return fail(HSTU_ERR_INVALID_ARG, "pair row %lld outside [0, T)", (long long)hp[i]);
  }
  st = device(hstu::launch_debug_indices(*desc, off, nc, B, T, ts, pairs, n, out, s), "debug launch");
  if (st != HSTU_OK) return st;
  return ok();
}

hstu_status hstu_debug_attn_bias(const hstu_desc* desc, const int64_t* off, int32_t B, int64_t T,
                                 const int64_t* ts, const int32_t* nc, const hstu_bias_tables* tables,
                                 const int32_t* slot, int32_t n_slots, int32_t max_len, float* out, void* ws,
                                 size_t ws_bytes, hstu_stream_t stream) {
  hstu_status st;
  if ((st = check_desc(desc)) != HSTU_OK) return st;
  if ((st = check_sizes(T, B)) != HSTU_OK) return st;
  if (desc->num_types > 0) return fail(HSTU_ERR_UNSUPPORTED, "bias inspection: token types not supported");
  if (n_slots < 0 || max_len < 0)
    return fail(HSTU_ERR_INVALID_ARG, "n_slots %d and max_len %d must be >= 0", n_slots, max_len);
  if (T == 0 || n_slots == 0 || max_len == 0) return ok();
  if ((st = check_meta(off, B, ts, nc)) != HSTU_OK) return st;
  if ((st = check_tables(desc, tables)) != HSTU_OK) return st;
  HSTU_REQ(slot, 4, "slot");
  HSTU_REQ(out, 4, "out");
  const size_t need = attn_ws(T, B);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return fail(HSTU_ERR_WORKSPACE, "workspace: need %zu bytes (256-aligned), got %zu", need, ws_bytes);
  hipStream_t s = (hipStream_t)stream;
  if (desc->flags & HSTU_VALIDATE)
    if ((st = validate_metadata(off, B, T, nc, s)) != HSTU_OK) return st;
  const hstu::AttnScratch sc = hstu::attn_scratch(ws, T, B);
  const hstu::AttnRows rows{off, nc, ts, T, off, ts, T, nullptr, B, false, {}};
  if ((st = device(hstu::launch_attn_prep(rows, hstu::kAttnBM, sc, s), "attention prep launch")) != HSTU_OK)
    return st;
  return device(hstu::launch_attn_dump(*desc, rows, *tables, slot, n_slots, max_len, out, sc, s),
                "bias inspection launch");
}

}  // extern "C"
