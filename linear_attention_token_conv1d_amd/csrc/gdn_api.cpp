// C ABI of the Gated DeltaNet token mixer: argument validation, error
// reporting and dispatch to the gfx950 kernel launchers.
//
// Every entry point validates its arguments completely before launching
// anything, so a rejected call writes nothing.  No C++ exception crosses the
// boundary.  GDN_DEBUG=1 in the environment makes every call synchronise its
// stream and report asynchronous kernel errors as GDN_ERR_HIP.
#include "../../include/gdn.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstddef>
#include <cstdio>
#include <cstdlib>
#include <string>

#include "gdn_internal.h"

namespace {

thread_local std::string g_last_error;

gdn_status fail(gdn_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool debug_sync() {
  static const bool on = [] {
    const char* e = std::getenv("GDN_DEBUG");
    return e && e[0] && e[0] != '0';
  }();
  return on;
}

gdn_status finish(hipError_t e, hipStream_t stream, const char* what) {
  if (e == hipSuccess && debug_sync()) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail(GDN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  g_last_error.clear();
  return GDN_OK;
}

bool is_dtype(int32_t d) { return d == GDN_F32 || d == GDN_BF16; }
size_t esize(int32_t d) { return d == GDN_BF16 ? 2 : 4; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || !na || !nb) return false;
  const char* x = static_cast<const char*>(a);
  const char* y = static_cast<const char*>(b);
  return x < y + nb && y < x + na;
}

// Fields added after ABI 3 read as their defaults from a shorter struct.
int32_t prefill_state_dtype(const gdn_prefill_args* a) {
  return a->struct_size >= sizeof(gdn_prefill_args) ? a->state_dtype : (int32_t)GDN_F32;
}
int32_t* conv_head_of(const gdn_conv1d_args* a) {
  return a->struct_size >= sizeof(gdn_conv1d_args) ? a->conv_head : nullptr;
}
int32_t* conv_head_of(const gdn_decode_args* a) {
  return a->struct_size >= sizeof(gdn_decode_args) ? a->conv_head : nullptr;
}

gdn_status check_prefill(const gdn_prefill_args* a, bool workspace = true) {
  if (!a) return fail(GDN_ERR_INVALID_ARG, "gdn_prefill: args is NULL");
  if (a->struct_size < offsetof(gdn_prefill_args, state_dtype))
    return fail(GDN_ERR_INVALID_ARG, "gdn_prefill: struct_size %u < %zu", a->struct_size,
                offsetof(gdn_prefill_args, state_dtype));
  if (!is_dtype(prefill_state_dtype(a)))
    return fail(GDN_ERR_INVALID_ARG, "gdn_prefill: bad state_dtype %d", prefill_state_dtype(a));
  if (!is_dtype(a->io_dtype)) return fail(GDN_ERR_INVALID_ARG, "gdn_prefill: bad io_dtype %d", a->io_dtype);
  if (a->flags & ~(GDN_FLAG_L2NORM_QK | GDN_FLAG_NO_ERASE))
    return fail(GDN_ERR_INVALID_ARG, "gdn_prefill: unknown flags 0x%x", a->flags);
  if (a->n_seqs < 1) return fail(GDN_ERR_INVALID_ARG, "gdn_prefill: n_seqs %d < 1", a->n_seqs);
  if (a->total_tokens < 0) return fail(GDN_ERR_INVALID_ARG, "gdn_prefill: total_tokens < 0");
  if (a->h_qk < 1 || a->h_v < 1 || a->h_v % a->h_qk)
    return fail(GDN_ERR_INVALID_ARG, "gdn_prefill: h_v (%d) must be a positive multiple of h_qk (%d)",
                a->h_v, a->h_qk);
  if (a->d_k != a->d_v || (a->d_k != 64 && a->d_k != 128))
    return fail(GDN_ERR_UNSUPPORTED, "gdn_prefill: d_k = d_v in {64, 128} required (got %d, %d)",
                a->d_k, a->d_v);
  if (a->chunk != 16 && a->chunk != 32 && a->chunk != 64)
    return fail(GDN_ERR_UNSUPPORTED, "gdn_prefill: chunk %d not in {16, 32, 64}", a->chunk);
  if (!gdn::prefill_supported(a->io_dtype, a->d_k, a->chunk))
    return fail(GDN_ERR_UNSUPPORTED, "gdn_prefill: io_dtype %d with d=%d and chunk %d exceeds LDS",
                a->io_dtype, a->d_k, a->chunk);
  if (a->total_tokens > 0 && (!a->q || !a->k || !a->v || !a->g || !a->beta || !a->o))
    return fail(GDN_ERR_INVALID_ARG, "gdn_prefill: q, k, v, g, beta and o are required");
  if (a->n_seqs > 1 && !a->cu_seqlens)
    return fail(GDN_ERR_INVALID_ARG, "gdn_prefill: cu_seqlens is required when n_seqs > 1");
  const int64_t hk = (int64_t)a->h_qk * a->d_k, hv = (int64_t)a->h_v * a->d_v;
  if (a->q_stride < hk || a->k_stride < hk || a->v_stride < hv)
    return fail(GDN_ERR_INVALID_ARG, "gdn_prefill: token strides smaller than a token's heads");
  if (a->q_stride % 8 || a->k_stride % 8 || a->v_stride % 8)
    return fail(GDN_ERR_ALIGNMENT, "gdn_prefill: token strides must be multiples of 8 elements");
  const void* ptrs16[] = {a->q, a->k, a->v, a->o, a->initial_state, a->final_state};
  for (const void* p : ptrs16)
    if (!aligned(p, 16)) return fail(GDN_ERR_ALIGNMENT, "gdn_prefill: tensors must be 16-byte aligned");
  if (a->initial_state && a->final_state && a->initial_state != a->final_state) {
    // the two pools may be the same buffer, but must not partly overlap
    const size_t ns = (size_t)a->n_seqs * a->h_v * a->d_v * a->d_k * esize(prefill_state_dtype(a));
    if (!a->state_idx && overlaps(a->initial_state, ns, a->final_state, ns))
      return fail(GDN_ERR_INVALID_ARG, "gdn_prefill: final_state partly overlaps initial_state");
  }
  if (!aligned(a->g, 4) || !aligned(a->beta, 4) || !aligned(a->cu_seqlens, 4))
    return fail(GDN_ERR_ALIGNMENT, "gdn_prefill: g, beta, cu_seqlens must be 4-byte aligned");
  if (a->emit_every < 0) return fail(GDN_ERR_INVALID_ARG, "gdn_prefill: emit_every %d < 0", a->emit_every);
  if (a->emit_every > 0 && a->total_tokens > 0 && !a->chunk_states)
    return fail(GDN_ERR_INVALID_ARG, "gdn_prefill: chunk_states is required when emit_every > 0");
  if (!aligned(a->chunk_states, 16) || !aligned(a->state_idx, 4))
    return fail(GDN_ERR_ALIGNMENT, "gdn_prefill: chunk_states must be 16-byte, state_idx 4-byte aligned");
  if (!workspace) return GDN_OK;
  const size_t need = gdn::prefill_workspace_bytes(a->io_dtype, a->total_tokens, a->n_seqs, a->h_v,
                                                   a->d_k, a->chunk, a->emit_every);
  if (need && (!a->workspace || a->workspace_bytes < need))
    return fail(GDN_ERR_WORKSPACE, "gdn_prefill: workspace of %zu bytes required", need);
  if (need && !aligned(a->workspace, 256))
    return fail(GDN_ERR_ALIGNMENT, "gdn_prefill: workspace must be 256-byte aligned");
  return GDN_OK;
}

gdn_status check_prefill_backward(const gdn_prefill_backward_args* a) {
  const char* f = "gdn_prefill_backward";
  if (!a) return fail(GDN_ERR_INVALID_ARG, "%s: args is NULL", f);
  if (a->struct_size < sizeof(gdn_prefill_backward_args))
    return fail(GDN_ERR_INVALID_ARG, "%s: struct_size %u < %zu", f, a->struct_size,
                sizeof(gdn_prefill_backward_args));
  if (!is_dtype(a->io_dtype)) return fail(GDN_ERR_INVALID_ARG, "%s: bad io_dtype %d", f, a->io_dtype);
  if (a->flags & ~(GDN_FLAG_L2NORM_QK | GDN_FLAG_NO_ERASE))
    return fail(GDN_ERR_INVALID_ARG, "%s: unknown flags 0x%x", f, a->flags);
  if (a->n_seqs < 1) return fail(GDN_ERR_INVALID_ARG, "%s: n_seqs %d < 1", f, a->n_seqs);
  if (a->total_tokens < 0 || a->total_tokens > INT32_MAX)
    return fail(GDN_ERR_INVALID_ARG, "%s: total_tokens out of range", f);
  if (a->h_qk < 1 || a->h_v < 1 || a->h_v % a->h_qk)
    return fail(GDN_ERR_INVALID_ARG, "%s: h_v (%d) must be a positive multiple of h_qk (%d)", f, a->h_v, a->h_qk);
  if (a->d_k != a->d_v || (a->d_k != 64 && a->d_k != 128))
    return fail(GDN_ERR_UNSUPPORTED, "%s: d_k = d_v in {64, 128} required (got %d, %d)", f, a->d_k, a->d_v);
  if (a->chunk != 16 && a->chunk != 32 && a->chunk != 64)
    return fail(GDN_ERR_UNSUPPORTED, "%s: chunk %d not in {16, 32, 64}", f, a->chunk);
  if (a->total_tokens > 0 && (!a->q || !a->k || !a->v || !a->g || !a->beta || !a->d_o || !a->dq || !a->dk ||
                              !a->dv || !a->dg || !a->dbeta))
    return fail(GDN_ERR_INVALID_ARG, "%s: q, k, v, g, beta, d_o, dq, dk, dv, dg and dbeta are required", f);
  if (a->n_seqs > 1 && !a->cu_seqlens)
    return fail(GDN_ERR_INVALID_ARG, "%s: cu_seqlens is required when n_seqs > 1", f);
  const int64_t hk = (int64_t)a->h_qk * a->d_k, hv = (int64_t)a->h_v * a->d_v;
  if (a->q_stride < hk || a->k_stride < hk || a->v_stride < hv || a->dq_stride < hk || a->dk_stride < hk ||
      a->dv_stride < hv)
    return fail(GDN_ERR_INVALID_ARG, "%s: token strides smaller than a token's heads", f);
  if ((a->q_stride | a->k_stride | a->v_stride | a->dq_stride | a->dk_stride | a->dv_stride) % 8)
    return fail(GDN_ERR_ALIGNMENT, "%s: token strides must be multiples of 8 elements", f);
  const void* ptrs16[] = {a->q, a->k, a->v, a->d_o, a->dq, a->dk, a->dv, a->initial_state, a->d_final_state,
                          a->d_initial_state};
  for (const void* p : ptrs16)
    if (!aligned(p, 16)) return fail(GDN_ERR_ALIGNMENT, "%s: tensors must be 16-byte aligned", f);
  if (!aligned(a->g, 4) || !aligned(a->beta, 4) || !aligned(a->cu_seqlens, 4) || !aligned(a->dg, 4) ||
      !aligned(a->dbeta, 4))
    return fail(GDN_ERR_ALIGNMENT, "%s: g, beta, dg, dbeta and cu_seqlens must be 4-byte aligned", f);
  // outputs must not overlap inputs (extents from the first to the last element)
  const size_t es = esize(a->io_dtype), T = (size_t)a->total_tokens;
  const size_t nS = (size_t)a->n_seqs * a->h_v * a->d_v * a->d_k * 4;
  auto span = [&](int64_t stride, int64_t width, size_t e) { return T ? ((T - 1) * stride + width) * e : 0; };
  struct R { const void* p; size_t n; };
  const R ins[] = {{a->q, span(a->q_stride, hk, es)}, {a->k, span(a->k_stride, hk, es)},
                   {a->v, span(a->v_stride, hv, es)}, {a->d_o, T * hv * es},
                   {a->g, T * a->h_v * 4}, {a->beta, T * a->h_v * 4},
                   {a->initial_state, a->initial_state ? nS : 0}, {a->d_final_state, a->d_final_state ? nS : 0}};
  const R outs[] = {{a->dq, span(a->dq_stride, hk, es)}, {a->dk, span(a->dk_stride, hk, es)},
                    {a->dv, span(a->dv_stride, hv, es)}, {a->dg, T * a->h_v * 4}, {a->dbeta, T * a->h_v * 4},
                    {a->d_initial_state, a->d_initial_state ? nS : 0}};
  for (const R& o : outs)
    for (const R& i : ins)
      if (overlaps(o.p, o.n, i.p, i.n)) return fail(GDN_ERR_INVALID_ARG, "%s: an output overlaps an input", f);
  const size_t need = gdn::prefill_backward_workspace_bytes(a->io_dtype, a->total_tokens, a->n_seqs, a->h_qk,
                                                            a->h_v, a->d_k,
                                                            a->chunk);
  if (!a->workspace || a->workspace_bytes < need)
    return fail(GDN_ERR_WORKSPACE, "%s: workspace of %zu bytes required", f, need);
  if (!aligned(a->workspace, 256)) return fail(GDN_ERR_ALIGNMENT, "%s: workspace must be 256-byte aligned", f);
  return GDN_OK;
}

gdn_status check_conv1d_backward(const gdn_conv1d_backward_args* a) {
  const char* f = "gdn_conv1d_backward";
  if (!a) return fail(GDN_ERR_INVALID_ARG, "%s: args is NULL", f);
  if (a->struct_size < sizeof(gdn_conv1d_backward_args))
    return fail(GDN_ERR_INVALID_ARG, "%s: struct_size %u < %zu", f, a->struct_size,
                sizeof(gdn_conv1d_backward_args));
  if (!is_dtype(a->dtype)) return fail(GDN_ERR_INVALID_ARG, "%s: bad dtype %d", f, a->dtype);
  if (a->n_seqs < 1) return fail(GDN_ERR_INVALID_ARG, "%s: n_seqs %d < 1", f, a->n_seqs);
  if (a->total_tokens < 0) return fail(GDN_ERR_INVALID_ARG, "%s: total_tokens < 0", f);
  if (a->channels < 8 || a->channels % 8)
    return fail(GDN_ERR_UNSUPPORTED, "%s: channels (%d) must be a positive multiple of 8", f, a->channels);
  if (a->width < 2 || a->width > 4) return fail(GDN_ERR_UNSUPPORTED, "%s: width %d not in 2..4", f, a->width);
  if (a->activation != GDN_ACT_NONE && a->activation != GDN_ACT_SILU)
    return fail(GDN_ERR_INVALID_ARG, "%s: bad activation %d", f, a->activation);
  if (!a->weight || !a->dweight || (a->total_tokens > 0 && (!a->x || !a->dy || !a->dx)))
    return fail(GDN_ERR_INVALID_ARG, "%s: x, weight, dy, dx and dweight are required", f);
  if (a->dbias && !a->bias) return fail(GDN_ERR_INVALID_ARG, "%s: dbias needs bias", f);
  if (a->n_seqs > 1 && !a->cu_seqlens)
    return fail(GDN_ERR_INVALID_ARG, "%s: cu_seqlens is required when n_seqs > 1", f);
  const size_t es = esize(a->dtype);
  if (!aligned(a->x, 16) || !aligned(a->dy, 16) || !aligned(a->dx, 16))
    return fail(GDN_ERR_ALIGNMENT, "%s: x, dy and dx must be 16-byte aligned", f);
  const void* pe[] = {a->weight, a->bias, a->conv_state};
  for (const void* p : pe)
    if (!aligned(p, es)) return fail(GDN_ERR_ALIGNMENT, "%s: misaligned tensor", f);
  const void* p4[] = {a->cu_seqlens, a->d_new_state, a->dweight, a->dbias, a->d_conv_state};
  for (const void* p : p4)
    if (!aligned(p, 4)) return fail(GDN_ERR_ALIGNMENT, "%s: misaligned fp32 or int32 tensor", f);
  const size_t TC = (size_t)a->total_tokens * a->channels;
  const size_t nS = (size_t)a->n_seqs * a->channels * (a->width - 1);
  struct R { const void* p; size_t n; };
  const R ins[] = {{a->x, TC * es}, {a->dy, TC * es}, {a->weight, (size_t)a->channels * a->width * es},
                   {a->bias, a->bias ? a->channels * es : 0}, {a->conv_state, a->conv_state ? nS * es : 0},
                   {a->d_new_state, a->d_new_state ? nS * 4 : 0}};
  const R outs[] = {{a->dx, TC * es}, {a->dweight, (size_t)a->channels * a->width * 4},
                    {a->dbias, a->dbias ? a->channels * 4u : 0}, {a->d_conv_state, a->d_conv_state ? nS * 4 : 0}};
  for (const R& o : outs)
    for (const R& i : ins)
      if (overlaps(o.p, o.n, i.p, i.n)) return fail(GDN_ERR_INVALID_ARG, "%s: an output overlaps an input", f);
  const size_t need = gdn::conv1d_backward_workspace_bytes(a->total_tokens, a->channels);
  if (!a->workspace || a->workspace_bytes < need)
    return fail(GDN_ERR_WORKSPACE, "%s: workspace of %zu bytes required", f, need);
  if (!aligned(a->workspace, 256)) return fail(GDN_ERR_ALIGNMENT, "%s: workspace must be 256-byte aligned", f);
  return GDN_OK;
}

}  // namespace

extern "C" {

const char* gdn_status_string(gdn_status s) {
  switch (s) {
    case GDN_OK: return "GDN_OK";
    case GDN_ERR_INVALID_ARG: return "GDN_ERR_INVALID_ARG";
    case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED";
    case GDN_ERR_ALIGNMENT: return "GDN_ERR_ALIGNMENT";
    case GDN_ERR_WORKSPACE: return "GDN_ERR_WORKSPACE";
    case GDN_ERR_HIP: return "GDN_ERR_HIP";
  }
  return "unknown gdn_status";
}

const char* gdn_last_error(void) { return g_last_error.c_str(); }

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

gdn_status gdn_conv1d(const gdn_conv1d_args* a, void* stream) {
  try {
    if (!a) return fail(GDN_ERR_INVALID_ARG, "gdn_conv1d: args is NULL");
    if (a->struct_size < offsetof(gdn_conv1d_args, conv_head))
      return fail(GDN_ERR_INVALID_ARG, "gdn_conv1d: struct_size %u < %zu", a->struct_size,
                  offsetof(gdn_conv1d_args, conv_head));
    if (!is_dtype(a->dtype)) return fail(GDN_ERR_INVALID_ARG, "gdn_conv1d: bad dtype %d", a->dtype);
    if (a->n_seqs < 1) return fail(GDN_ERR_INVALID_ARG, "gdn_conv1d: n_seqs %d < 1", a->n_seqs);
    if (a->total_tokens < 0) return fail(GDN_ERR_INVALID_ARG, "gdn_conv1d: total_tokens < 0");
    if (a->channels < 8 || a->channels % 8)
      return fail(GDN_ERR_UNSUPPORTED, "gdn_conv1d: channels (%d) must be a positive multiple of 8",
                  a->channels);
    if (a->width < 2 || a->width > 4)
      return fail(GDN_ERR_UNSUPPORTED, "gdn_conv1d: width %d not in 2..4", a->width);
    if (a->activation != GDN_ACT_NONE && a->activation != GDN_ACT_SILU)
      return fail(GDN_ERR_INVALID_ARG, "gdn_conv1d: bad activation %d", a->activation);
    if (!a->weight || (a->total_tokens > 0 && (!a->x || !a->y)))
      return fail(GDN_ERR_INVALID_ARG, "gdn_conv1d: x, weight and y are required");
    if (a->n_seqs > 1 && !a->cu_seqlens)
      return fail(GDN_ERR_INVALID_ARG, "gdn_conv1d: cu_seqlens is required when n_seqs > 1");
    if (!aligned(a->x, 16) || !aligned(a->y, 16))
      return fail(GDN_ERR_ALIGNMENT, "gdn_conv1d: x and y must be 16-byte aligned");
    if (!aligned(a->weight, esize(a->dtype)) || !aligned(a->bias, esize(a->dtype)) ||
        !aligned(a->conv_state, esize(a->dtype)) || !aligned(a->cu_seqlens, 4) ||
        !aligned(conv_head_of(a), 4))
      return fail(GDN_ERR_ALIGNMENT, "gdn_conv1d: misaligned weight, bias, conv_state, cu_seqlens or conv_head");
    const size_t bytes = (size_t)a->total_tokens * a->channels * esize(a->dtype);
    const char* xb = static_cast<const char*>(a->x);
    const char* yb = static_cast<const char*>(a->y);
    if (bytes && xb < yb + bytes && yb < xb + bytes)
      return fail(GDN_ERR_INVALID_ARG, "gdn_conv1d: y must not overlap x");
    gdn::ConvParams p{a->x, a->weight, a->bias, a->y, a->conv_state, a->cu_seqlens,
                      a->total_tokens, a->n_seqs, a->channels, a->width, a->activation,
                      a->conv_state ? conv_head_of(a) : nullptr};
    hipStream_t s = static_cast<hipStream_t>(stream);
    return finish(gdn::launch_conv1d(p, a->dtype, s), s, "gdn_conv1d");
  } catch (...) {
    return fail(GDN_ERR_HIP, "gdn_conv1d: internal error");
  }
}

size_t gdn_prefill_workspace_size(const gdn_prefill_args* a) {
  if (!a || a->struct_size < offsetof(gdn_prefill_args, state_dtype)) return 0;
  return gdn::prefill_workspace_bytes(a->io_dtype, a->total_tokens, a->n_seqs, a->h_v, a->d_k, a->chunk,
                                      a->emit_every > 0 ? a->emit_every : 0);
}

static_assert(GDN_NOALLOC_MAX_SEQS == gdn::kNoAllocMaxSeqs, "static plan size");

namespace {
gdn::PrefillParams prefill_params(const gdn_prefill_args* a) {
  return gdn::PrefillParams{a->q, a->k, a->v, a->q_stride, a->k_stride, a->v_stride,
                            a->g, a->beta, a->initial_state, a->final_state, a->o, a->cu_seqlens,
                            a->total_tokens, a->n_seqs, a->h_qk, a->h_v, a->chunk,
                            (a->flags & GDN_FLAG_L2NORM_QK) ? 1 : 0, a->scale, a->workspace,
                            a->workspace_bytes, (a->flags & GDN_FLAG_NO_ERASE) ? 0 : 1, a->emit_every,
                            a->chunk_states, a->state_idx, prefill_state_dtype(a) == GDN_BF16 ? 1 : 0};
}
}  // namespace

gdn_status gdn_prefill_noalloc(const gdn_prefill_args* a, void* stream) {
  try {
    gdn_status st = check_prefill(a, false);
    if (st != GDN_OK) return st;
    if (a->io_dtype != GDN_BF16 || (a->chunk != 32 && a->chunk != 64))
      return fail(GDN_ERR_UNSUPPORTED, "gdn_prefill_noalloc: bf16 io at chunk 32 or 64 required (got io_dtype %d, "
                  "chunk %d)", a->io_dtype, a->chunk);
    if (a->n_seqs > GDN_NOALLOC_MAX_SEQS)
      return fail(GDN_ERR_INVALID_ARG, "gdn_prefill_noalloc: n_seqs %d exceeds the static plan's %d sequences",
                  a->n_seqs, GDN_NOALLOC_MAX_SEQS);
    hipStream_t s = static_cast<hipStream_t>(stream);
    return finish(gdn::launch_prefill_noalloc(prefill_params(a), a->d_k, s), s, "gdn_prefill_noalloc");
  } catch (...) {
    return fail(GDN_ERR_HIP, "gdn_prefill_noalloc: internal error");
  }
}

gdn_status gdn_prefill(const gdn_prefill_args* a, void* stream) {
  try {
    gdn_status st = check_prefill(a);
    if (st != GDN_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return finish(gdn::launch_prefill(prefill_params(a), a->io_dtype, a->d_k, s), s, "gdn_prefill");
  } catch (...) {
    return fail(GDN_ERR_HIP, "gdn_prefill: internal error");
  }
}

gdn_status gdn_decode_step(const gdn_decode_args* a, void* stream) {
  try {
    if (!a) return fail(GDN_ERR_INVALID_ARG, "gdn_decode_step: args is NULL");
    if (a->struct_size < offsetof(gdn_decode_args, conv_head))
      return fail(GDN_ERR_INVALID_ARG, "gdn_decode_step: struct_size %u < %zu", a->struct_size,
                  offsetof(gdn_decode_args, conv_head));
    if (!is_dtype(a->io_dtype) || !is_dtype(a->state_dtype))
      return fail(GDN_ERR_INVALID_ARG, "gdn_decode_step: bad io_dtype/state_dtype");
    if (a->flags & ~(GDN_FLAG_L2NORM_QK | GDN_FLAG_NO_ERASE))
      return fail(GDN_ERR_INVALID_ARG, "gdn_decode_step: unknown flags 0x%x", a->flags);
    if (a->n_seqs < 0) return fail(GDN_ERR_INVALID_ARG, "gdn_decode_step: n_seqs < 0");
    if (a->h_qk < 1 || a->h_v < 1 || a->h_v % a->h_qk)
      return fail(GDN_ERR_INVALID_ARG, "gdn_decode_step: h_v (%d) must be a positive multiple of h_qk (%d)",
                  a->h_v, a->h_qk);
    if (a->h_v / a->h_qk > 16)
      return fail(GDN_ERR_UNSUPPORTED, "gdn_decode_step: more than 16 V heads per QK head");
    if (a->d_k != a->d_v || (a->d_k != 64 && a->d_k != 128))
      return fail(GDN_ERR_UNSUPPORTED, "gdn_decode_step: d_k = d_v in {64, 128} required");
    if (a->conv_weight && (a->width < 2 || a->width > 4))
      return fail(GDN_ERR_UNSUPPORTED, "gdn_decode_step: width %d not in 2..4", a->width);
    if (a->activation != GDN_ACT_NONE && a->activation != GDN_ACT_SILU)
      return fail(GDN_ERR_INVALID_ARG, "gdn_decode_step: bad activation %d", a->activation);
    if (a->n_seqs > 0 && (!a->x || !a->g || !a->beta || !a->state || !a->o))
      return fail(GDN_ERR_INVALID_ARG, "gdn_decode_step: x, g, beta, state and o are required");
    if (a->n_seqs > 0 && a->conv_weight && !a->conv_state)
      return fail(GDN_ERR_INVALID_ARG, "gdn_decode_step: conv_state is required with a conv");
    if (!aligned(a->state, 16))
      return fail(GDN_ERR_ALIGNMENT, "gdn_decode_step: state must be 16-byte aligned");
    if (!aligned(a->state_idx, 4) || !aligned(conv_head_of(a), 4))
      return fail(GDN_ERR_ALIGNMENT, "gdn_decode_step: state_idx and conv_head must be 4-byte aligned");
    const size_t es = esize(a->io_dtype);
    if (!aligned(a->x, es) || !aligned(a->o, es) || !aligned(a->conv_weight, es) ||
        !aligned(a->conv_bias, es) || !aligned(a->conv_state, es) || !aligned(a->g, 4) ||
        !aligned(a->beta, 4))
      return fail(GDN_ERR_ALIGNMENT, "gdn_decode_step: misaligned tensor");
    if (a->n_seqs == 0) { g_last_error.clear(); return GDN_OK; }
    gdn::DecodeParams p{a->x, a->conv_weight, a->conv_bias, a->conv_state, a->g, a->beta,
                        a->state, a->o, a->n_seqs, a->h_qk, a->h_v, a->conv_weight ? a->width : 4,
                        a->activation, (a->flags & GDN_FLAG_L2NORM_QK) ? 1 : 0, a->scale,
                        (a->flags & GDN_FLAG_NO_ERASE) ? 0 : 1, a->state_idx,
                        a->conv_weight ? conv_head_of(a) : nullptr};
    hipStream_t s = static_cast<hipStream_t>(stream);
    return finish(gdn::launch_decode(p, a->io_dtype, a->state_dtype, a->d_k, s), s, "gdn_decode_step");
  } catch (...) {
    return fail(GDN_ERR_HIP, "gdn_decode_step: internal error");
  }
}

size_t gdn_prefill_backward_workspace_size(const gdn_prefill_backward_args* a) {
  if (!a || a->struct_size < sizeof(gdn_prefill_backward_args) || a->n_seqs < 1 || a->total_tokens < 0 ||
      a->h_qk < 1 || a->h_v < 1 || a->h_v % a->h_qk || a->d_k != a->d_v || (a->d_k != 64 && a->d_k != 128) ||
      (a->chunk != 16 && a->chunk != 32 && a->chunk != 64))
    return 0;
  return gdn::prefill_backward_workspace_bytes(a->io_dtype, a->total_tokens, a->n_seqs, a->h_qk, a->h_v, a->d_k,
                                               a->chunk);
}

gdn_status gdn_prefill_backward(const gdn_prefill_backward_args* a, void* stream) {
  try {
    const gdn_status s = check_prefill_backward(a);
    if (s != GDN_OK) return s;
    gdn::PrefillBwdParams p{a->q, a->k, a->v, a->q_stride, a->k_stride, a->v_stride, a->g, a->beta,
                            a->initial_state, a->cu_seqlens, a->d_o, a->d_final_state, a->dq, a->dk, a->dv,
                            a->dq_stride, a->dk_stride, a->dv_stride, a->dg, a->dbeta, a->d_initial_state,
                            a->total_tokens, a->n_seqs, a->h_qk, a->h_v, a->chunk,
                            (a->flags & GDN_FLAG_L2NORM_QK) ? 1 : 0, (a->flags & GDN_FLAG_NO_ERASE) ? 0 : 1,
                            a->scale, a->workspace};
    hipStream_t st = static_cast<hipStream_t>(stream);
    return finish(gdn::launch_prefill_backward(p, a->io_dtype, a->d_k, st), st, "gdn_prefill_backward");
  } catch (...) {
    return fail(GDN_ERR_HIP, "gdn_prefill_backward: internal error");
  }
}

size_t gdn_conv1d_backward_workspace_size(const gdn_conv1d_backward_args* a) {
  if (!a || a->struct_size < sizeof(gdn_conv1d_backward_args) || a->total_tokens < 0 || a->channels < 8 ||
      a->channels % 8)
    return 0;
  return gdn::conv1d_backward_workspace_bytes(a->total_tokens, a->channels);
}

gdn_status gdn_conv1d_backward(const gdn_conv1d_backward_args* a, void* stream) {
  try {
    const gdn_status s = check_conv1d_backward(a);
    if (s != GDN_OK) return s;
    gdn::ConvBwdParams p{a->x, a->weight, a->bias, a->conv_state, a->cu_seqlens, a->dy, a->d_new_state, a->dx,
                         a->dweight, a->dbias, a->d_conv_state, a->total_tokens, a->n_seqs, a->channels,
                         a->width, a->activation, a->workspace};
    hipStream_t st = static_cast<hipStream_t>(stream);
    return finish(gdn::launch_conv1d_backward(p, a->dtype, st), st, "gdn_conv1d_backward");
  } catch (...) {
    return fail(GDN_ERR_HIP, "gdn_conv1d_backward: internal error");
  }
}

}  // extern "C"
