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

gdn_status check_prefill(const gdn_prefill_args* a) {
  if (!a) return fail(GDN_ERR_INVALID_ARG, "gdn_prefill: args is NULL");
  if (a->struct_size < sizeof(gdn_prefill_args))
    return fail(GDN_ERR_INVALID_ARG, "gdn_prefill: struct_size %u < %zu", a->struct_size,
                sizeof(gdn_prefill_args));
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
  if (!aligned(a->g, 4) || !aligned(a->beta, 4) || !aligned(a->cu_seqlens, 4))
    return fail(GDN_ERR_ALIGNMENT, "gdn_prefill: g, beta, cu_seqlens must be 4-byte aligned");
  if (a->emit_every < 0) return fail(GDN_ERR_INVALID_ARG, "gdn_prefill: emit_every %d < 0", a->emit_every);
  if (a->emit_every > 0 && a->total_tokens > 0 && !a->chunk_states)
    return fail(GDN_ERR_INVALID_ARG, "gdn_prefill: chunk_states is required when emit_every > 0");
  if (!aligned(a->chunk_states, 16) || !aligned(a->state_idx, 4))
    return fail(GDN_ERR_ALIGNMENT, "gdn_prefill: chunk_states must be 16-byte, state_idx 4-byte aligned");
  const size_t need = gdn::prefill_workspace_bytes(a->io_dtype, a->total_tokens, a->n_seqs, a->h_v,
                                                   a->d_k, a->chunk, a->emit_every);
  if (need && (!a->workspace || a->workspace_bytes < need))
    return fail(GDN_ERR_WORKSPACE, "gdn_prefill: workspace of %zu bytes required", need);
  if (need && !aligned(a->workspace, 256))
    return fail(GDN_ERR_ALIGNMENT, "gdn_prefill: workspace must be 256-byte aligned");
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
    if (a->struct_size < sizeof(gdn_conv1d_args))
      return fail(GDN_ERR_INVALID_ARG, "gdn_conv1d: struct_size %u < %zu", a->struct_size,
                  sizeof(gdn_conv1d_args));
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
        !aligned(a->conv_state, esize(a->dtype)) || !aligned(a->cu_seqlens, 4))
      return fail(GDN_ERR_ALIGNMENT, "gdn_conv1d: misaligned weight, bias, conv_state or cu_seqlens");
    const size_t bytes = (size_t)a->total_tokens * a->channels * esize(a->dtype);
    const char* xb = static_cast<const char*>(a->x);
    const char* yb = static_cast<const char*>(a->y);
    if (bytes && xb < yb + bytes && yb < xb + bytes)
      return fail(GDN_ERR_INVALID_ARG, "gdn_conv1d: y must not overlap x");
    gdn::ConvParams p{a->x, a->weight, a->bias, a->y, a->conv_state, a->cu_seqlens,
                      a->total_tokens, a->n_seqs, a->channels, a->width, a->activation};
    hipStream_t s = static_cast<hipStream_t>(stream);
    return finish(gdn::launch_conv1d(p, a->dtype, s), s, "gdn_conv1d");
  } catch (...) {
    return fail(GDN_ERR_HIP, "gdn_conv1d: internal error");
  }
}

size_t gdn_prefill_workspace_size(const gdn_prefill_args* a) {
  if (!a || a->struct_size < sizeof(gdn_prefill_args)) return 0;
  return gdn::prefill_workspace_bytes(a->io_dtype, a->total_tokens, a->n_seqs, a->h_v, a->d_k, a->chunk,
                                      a->emit_every > 0 ? a->emit_every : 0);
}

gdn_status gdn_prefill(const gdn_prefill_args* a, void* stream) {
  try {
    gdn_status st = check_prefill(a);
    if (st != GDN_OK) return st;
    gdn::PrefillParams p{a->q, a->k, a->v, a->q_stride, a->k_stride, a->v_stride,
                         a->g, a->beta, a->initial_state, a->final_state, a->o, a->cu_seqlens,
                         a->total_tokens, a->n_seqs, a->h_qk, a->h_v, a->chunk,
                         (a->flags & GDN_FLAG_L2NORM_QK) ? 1 : 0, a->scale, a->workspace,
                         a->workspace_bytes, (a->flags & GDN_FLAG_NO_ERASE) ? 0 : 1, a->emit_every,
                         a->chunk_states, a->state_idx};
    hipStream_t s = static_cast<hipStream_t>(stream);
    return finish(gdn::launch_prefill(p, a->io_dtype, a->d_k, s), s, "gdn_prefill");
  } catch (...) {
    return fail(GDN_ERR_HIP, "gdn_prefill: internal error");
  }
}

gdn_status gdn_decode_step(const gdn_decode_args* a, void* stream) {
  try {
    if (!a) return fail(GDN_ERR_INVALID_ARG, "gdn_decode_step: args is NULL");
    if (a->struct_size < sizeof(gdn_decode_args))
      return fail(GDN_ERR_INVALID_ARG, "gdn_decode_step: struct_size %u < %zu", a->struct_size,
                  sizeof(gdn_decode_args));
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
    if (!aligned(a->state_idx, 4))
      return fail(GDN_ERR_ALIGNMENT, "gdn_decode_step: state_idx must be 4-byte aligned");
    const size_t es = esize(a->io_dtype);
    if (!aligned(a->x, es) || !aligned(a->o, es) || !aligned(a->conv_weight, es) ||
        !aligned(a->conv_bias, es) || !aligned(a->conv_state, es) || !aligned(a->g, 4) ||
        !aligned(a->beta, 4))
      return fail(GDN_ERR_ALIGNMENT, "gdn_decode_step: misaligned tensor");
    if (a->n_seqs == 0) { g_last_error.clear(); return GDN_OK; }
    gdn::DecodeParams p{a->x, a->conv_weight, a->conv_bias, a->conv_state, a->g, a->beta,
                        a->state, a->o, a->n_seqs, a->h_qk, a->h_v, a->conv_weight ? a->width : 4,
                        a->activation, (a->flags & GDN_FLAG_L2NORM_QK) ? 1 : 0, a->scale,
                        (a->flags & GDN_FLAG_NO_ERASE) ? 0 : 1, a->state_idx};
    hipStream_t s = static_cast<hipStream_t>(stream);
    return finish(gdn::launch_decode(p, a->io_dtype, a->state_dtype, a->d_k, s), s, "gdn_decode_step");
  } catch (...) {
    return fail(GDN_ERR_HIP, "gdn_decode_step: internal error");
  }
}

}  // extern "C"
