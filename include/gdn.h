/*
 * gdn.h -- C ABI of the Gated DeltaNet token mixer library for MI355X (gfx950).
 *
 * The mixer ("Inside Qwen3.5: a hybrid linear + full attention LLM",
 * sections 4-5 and the config note) is:
 *   1. a causal depthwise convolution of width 4 over the concatenated
 *      [q | k | v] channels, followed by SiLU;
 *   2. L2 normalisation of q and k per head;
 *   3. the gated delta rule per V head h (QK head h / (h_v / h_qk)):
 *        S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *        o_t = scale * S_t q_t,   alpha_t = exp(g_t),
 *      with a fixed d_v x d_k state per V head, updated in place.
 *   Decode is the same recurrence applied one token at a time: a
 *   read-modify-write of the fixed-size state ("Inside Qwen3.5", section 8).
 *
 * Conventions shared by every entry point
 *   - All tensor arguments are DEVICE pointers, row-major and contiguous
 *     unless a stride argument says otherwise.  The caller allocates and owns
 *     every buffer; the library allocates nothing and keeps no global mutable
 *     state other than a thread-local error string.
 *   - Every call is asynchronous and ordered on the given HIP stream
 *     (0 = the null stream).  Nothing is synchronised implicitly.
 *   - Each call takes a pointer to an argument struct whose first field is
 *     struct_size (set it to sizeof the struct).
 *   - Validation errors return before anything is launched and write
 *     nothing.  A failed launch returns GDN_ERR_HIP; gdn_last_error() gives
 *     the detail.  No C++ exception crosses this boundary.
 *   - Identical inputs give bitwise identical outputs (no atomics in any
 *     reduction).
 *   - Token counts and element offsets are 64-bit.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 4

typedef enum gdn_status {
  GDN_OK = 0,
  GDN_ERR_INVALID_ARG = 1, /* null pointer, bad size or shape            */
  GDN_ERR_UNSUPPORTED = 2, /* valid but not implemented (e.g. d_k = 96)  */
  GDN_ERR_ALIGNMENT = 3,   /* a pointer or stride breaks the alignment rule */
  GDN_ERR_WORKSPACE = 4,   /* workspace missing or too small             */
  GDN_ERR_HIP = 5          /* the HIP runtime reported an error          */
} gdn_status;

typedef enum gdn_dtype { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

typedef enum gdn_activation { GDN_ACT_NONE = 0, GDN_ACT_SILU = 1 } gdn_activation;

/* flags */
#define GDN_FLAG_L2NORM_QK 1u /* L2-normalise q and k per head (eps 1e-6 inside the sqrt) */
/* Erase-off variant: S_t = a_t S_{t-1} + b_t v_t k_t^T, the additive linear
 * attention of "Inside Qwen3.5", section 2 (S = sum v k^T, o = S q) with the
 * decay gate of section 5 kept and its error-correcting write dropped. */
#define GDN_FLAG_NO_ERASE 2u

/* ------------------------------------------------------------------------
 * gdn_conv1d -- causal depthwise convolution (+ optional SiLU) over packed
 * sequences, with a per-sequence conv state.
 *
 * Defined by "Inside Qwen3.5", section 5 (a kernel-4 causal convolution ahead
 * of the recurrence) and "Mamba hybrid model selection", per-request memory
 * section (a (channels, kernel width - 1) conv state per sequence):
 *   y[t, c] = act( sum_{j<W} w[c, j] * x[t - (W-1) + j, c] + bias[c] )
 * where inputs before a sequence's first token come from that sequence's
 * conv state (oldest first), or are zero when conv_state is NULL.
 *
 *   dtype        GDN_BF16 or GDN_F32: dtype of x, weight, bias, y, conv_state
 *                (accumulation is fp32).
 *   n_seqs       number of packed sequences (>= 1).
 *   total_tokens T, sum of the sequence lengths (>= 0).
 *   channels     C (multiple of 8).
 *   width        W, 2..4.
 *   activation   GDN_ACT_NONE or GDN_ACT_SILU.
 *   x            [T, C] input, 16-byte aligned.
 *   weight       [C, W].
 *   bias         [C] or NULL.
 *   y            [T, C] output; must not overlap x.
 *   conv_state   [n_seqs, C, W-1] in/out, or NULL.  On return it holds the
 *                last W-1 inputs of (old state ++ sequence), oldest first
 *                (chronological: slot 0 the oldest); a zero-length sequence
 *                keeps its inputs.
 *   cu_seqlens   [n_seqs + 1] int32 device array of sequence offsets
 *                (0 = cu[0] <= cu[1] <= ... = T), or NULL for one sequence.
 *                Values are trusted (not validated on the host).
 *   conv_head    [n_seqs] int32 ring heads of conv_state, or NULL.  With a
 *                head h, the state's W-1 slots form a ring: the j-th oldest
 *                input sits in slot (h + j) mod (W-1), so that a decode step
 *                can replace one slot instead of shifting all of them (the
 *                conv state is a fixed (channels, width - 1) buffer per
 *                request, "Mamba hybrid model selection", per-request memory
 *                section).  On entry 0 <= h < W-1 (taken mod W-1); on return
 *                the state is chronological and every head is 0.  NULL means
 *                chronological on entry.  Ignored without conv_state.  The
 *                library uses the bits above the lowest 8 of each head as a
 *                reader count during the call: nothing else may access
 *                conv_head until the call has finished on the stream.
 * Structs from callers built against ABI 3 (struct_size without conv_head)
 * are accepted and read as conv_head = NULL.
 * ---------------------------------------------------------------------- */
typedef struct gdn_conv1d_args {
  uint32_t struct_size;
  int32_t dtype;
  int32_t n_seqs;
  int32_t channels;
  int64_t total_tokens;
  int32_t width;
  int32_t activation;
  const void* x;
  const void* weight;
  const void* bias;
  void* y;
  void* conv_state;
  const int32_t* cu_seqlens;
  int32_t* conv_head;
} gdn_conv1d_args;

gdn_status gdn_conv1d(const gdn_conv1d_args* args, void* stream);

/* ------------------------------------------------------------------------
 * gdn_prefill -- chunked gated delta rule over packed sequences.
 *
 * Computes, for every sequence and V head, the recurrence stated at the top
 * of this file ("Inside Qwen3.5", sections 4-5), exactly up to rounding, by
 * the chunked WY / UT-transform rearrangement (chunks restart at each
 * sequence start; the last chunk may be partial).
 *
 *   io_dtype     GDN_BF16 or GDN_F32: dtype of q, k, v and o.  The state is
 *                carried in fp32 inside the call; accumulation is fp32.  With
 *                GDN_BF16 the dense chunk contractions run on bf16 MFMA; with
 *                GDN_F32 on fp32 MFMA.
 *   flags        GDN_FLAG_L2NORM_QK to normalise q and k inside the call;
 *                GDN_FLAG_NO_ERASE for the erase-off variant (same chunked
 *                machinery with A = 0, i.e. T = I, and U = diag(beta) V).
 *   n_seqs       >= 1.    total_tokens T >= 0.
 *   h_qk, h_v    head counts, h_v % h_qk == 0.
 *   d_k, d_v     head widths: both 64 or both 128.
 *   chunk        16, 32 or 64.
 *   scale        output scale (1.0 reproduces o = S q).
 *   q, k         [T, h_qk, d_k] with token stride q_stride / k_stride
 *                (elements; heads contiguous inside a token).  q, k and v may
 *                be column slices of the conv output [T, C].
 *   v            [T, h_v, d_v] with token stride v_stride.
 *   g, beta      [T, h_v] fp32: log-decay (alpha = exp(g) in (0, 1]) and
 *                write strength.
 *   initial_state [n_seqs, h_v, d_v, d_k] in state_dtype, or NULL for zeros.
 *   final_state  [n_seqs, h_v, d_v, d_k] in state_dtype, or NULL; may alias
 *                initial_state.
 *   o            [T, h_v, d_v] in io_dtype.
 *   cu_seqlens   as in gdn_conv1d.
 *   workspace    device scratch of at least gdn_prefill_workspace_size()
 *                bytes, 256-byte aligned.  Contents on entry are ignored.
 *   emit_every   K >= 0.  With K > 0 the state after every K-th whole chunk
 *                of a sequence that ends before the sequence does (tokens
 *                j K chunk, j = 1, 2, ..., strictly inside the sequence) is
 *                written to chunk_states, for prefix caching: the chunk
 *                boundary states already exist on chip, and a recurrent cache
 *                can be reused only from states stored at block boundaries
 *                ("Mamba hybrid model selection", adoption checklist).
 *   chunk_states [R, h_v, d_v, d_k] in state_dtype, R = sum_n E_n with
 *                E_n = floor(max(len_n - 1, 0) / (K chunk)); sequence n's
 *                states are rows sum_{m<n} E_m + j - 1.  NULL when K = 0.
 *   state_idx    [n_seqs] int32 or NULL: sequence n reads initial_state and
 *                writes final_state at slot state_idx[n] of [slots, h_v, d_v,
 *                d_k] pools (NULL: slot n), for caches that keep states in
 *                slots across requests ("Mamba hybrid model selection",
 *                concurrent-requests section).  Slots must be distinct and
 *                inside both pools; they are not read on the host.
 *   state_dtype  GDN_F32 or GDN_BF16: dtype of initial_state, final_state
 *                and chunk_states in memory.  The model keeps its recurrent
 *                state in fp32 ("Inside Qwen3.5", config note); a bf16 pool
 *                halves the bytes a decode step moves ("Mamba hybrid model
 *                selection", adoption checklist: the state's precision is a
 *                choice).  bf16 states are read exactly and written with
 *                round-to-nearest-even; inside the call the state is fp32.
 * Structs from callers built against ABI 3 (struct_size without state_dtype)
 * are accepted and read as state_dtype = GDN_F32.
 * ---------------------------------------------------------------------- */
typedef struct gdn_prefill_args {
  uint32_t struct_size;
  uint32_t flags;
  int32_t io_dtype;
  int32_t n_seqs;
  int64_t total_tokens;
  int32_t h_qk;
  int32_t h_v;
  int32_t d_k;
  int32_t d_v;
  int32_t chunk;
  float scale;
  const void* q;
  const void* k;
  const void* v;
  int64_t q_stride;
  int64_t k_stride;
  int64_t v_stride;
  const float* g;
  const float* beta;
  const void* initial_state;
  void* final_state;
  void* o;
  const int32_t* cu_seqlens;
  void* workspace;
  size_t workspace_bytes;
  int32_t emit_every;
  void* chunk_states;
  const int32_t* state_idx;
  int32_t state_dtype;
} gdn_prefill_args;

/* Bytes of workspace gdn_prefill needs for these arguments (pointers are not
 * read).  Returns 0 when the arguments are invalid. */
size_t gdn_prefill_workspace_size(const gdn_prefill_args* args);

gdn_status gdn_prefill(const gdn_prefill_args* args, void* stream);

/* gdn_prefill_noalloc -- gdn_prefill that allocates nothing and takes no
 * workspace, for callers that cannot allocate device memory (code under
 * stream capture, serving loops and harnesses that forbid allocation).
 * Same arguments and results as gdn_prefill, restricted to io_dtype GDN_BF16
 * at chunk 32 or 64 (the fused kernel; else GDN_ERR_UNSUPPORTED) and n_seqs
 * <= GDN_NOALLOC_MAX_SEQS (else GDN_ERR_INVALID_ARG); workspace and
 * workspace_bytes are ignored.  The per-call plan (chunk offsets, scan order,
 * emitted-state rows) lives in a static device array of about 96 KiB, one per
 * GPU, held until the process ends and shared by every call on that GPU:
 * calls that overlap on one GPU (concurrent streams or threads) race. */
#define GDN_NOALLOC_MAX_SEQS 8192
gdn_status gdn_prefill_noalloc(const gdn_prefill_args* args, void* stream);

/* ------------------------------------------------------------------------
 * gdn_decode_step -- one new token for each of n_seqs independent sequences.
 *
 * Fuses, per sequence: the conv step over the new token (reading the W-1
 * stored inputs, then storing the new input in the conv state), SiLU, the
 * split into [q | k | v], the optional L2 norm, and one step of the gated
 * delta rule on that sequence's state, which is read once and written once
 * ("Inside Qwen3.5", section 8: decode is a read-modify-write of the
 * fixed-size state every token; "Mamba hybrid model selection", decode
 * section: the step is bounded by the bytes it moves over HBM bandwidth).
 *
 *   io_dtype     GDN_BF16 or GDN_F32: dtype of x, conv_weight, conv_bias,
 *                conv_state and o.
 *   state_dtype  GDN_BF16 (stored with round-to-nearest-even, accumulated in
 *                fp32) or GDN_F32.
 *   flags        GDN_FLAG_L2NORM_QK; GDN_FLAG_NO_ERASE for the erase-off
 *                variant (delta_i = beta v_i: the state is still read and
 *                written once).
 *   n_seqs       >= 0.   h_qk, h_v (h_v % h_qk == 0), d_k = d_v in {64, 128}.
 *   width        conv width W in 2..4 (ignored without conv_weight).
 *   activation   GDN_ACT_SILU or GDN_ACT_NONE.
 *   scale        output scale.
 *   x            [n_seqs, C] new inputs, C = 2 h_qk d_k + h_v d_v.
 *   conv_weight  [C, W], or NULL: then x already holds q|k|v (no conv, no
 *                activation, conv_state unused).
 *   conv_bias    [C] or NULL.
 *   conv_state   [n_seqs, C, W-1] in/out; required with a conv.  Without a
 *                ring head it is chronological (slot 0 the oldest) and the
 *                step shifts the new input in; with one, see conv_head.
 *   conv_head    [n_seqs] int32 ring heads, or NULL (chronological).  The
 *                j-th oldest input sits in slot (h + j) mod (W-1); the step
 *                reads the W-1 slots in that order, overwrites only slot h
 *                (the oldest) with the new input and sets the head to
 *                (h + 1) mod (W-1): one slot written per step instead of W-1
 *                ("Mamba hybrid model selection", per-request memory
 *                section: a fixed (channels, width - 1) conv buffer per
 *                request).  Indexed like conv_state (by state_idx when given).
 *                On entry 0 <= h < W-1 (taken mod W-1).  As in gdn_conv1d,
 *                the bits above the lowest 8 count readers during the call.
 *   g, beta      [n_seqs, h_v] fp32.
 *   state        [n_seqs, h_v, d_v, d_k] in/out, in state_dtype.
 *   o            [n_seqs, h_v, d_v] in io_dtype.
 *   state_idx    [n_seqs] int32 or NULL: sequence n's state and conv_state
 *                are slot state_idx[n] of [slots, ...] pools (NULL: slot n);
 *                x, g, beta and o stay indexed by n.  Slots must be distinct
 *                and inside both pools; they are not read on the host.
 * Structs from callers built against ABI 3 (struct_size without conv_head)
 * are accepted and read as conv_head = NULL.
 * ---------------------------------------------------------------------- */
typedef struct gdn_decode_args {
  uint32_t struct_size;
  uint32_t flags;
  int32_t io_dtype;
  int32_t state_dtype;
  int32_t n_seqs;
  int32_t h_qk;
  int32_t h_v;
  int32_t d_k;
  int32_t d_v;
  int32_t width;
  int32_t activation;
  float scale;
  const void* x;
  const void* conv_weight;
  const void* conv_bias;
  void* conv_state;
  const float* g;
  const float* beta;
  void* state;
  void* o;
  const int32_t* state_idx;
  int32_t* conv_head;
} gdn_decode_args;

gdn_status gdn_decode_step(const gdn_decode_args* args, void* stream);

/* ------------------------------------------------------------------------
 * gdn_prefill_backward -- gradients of gdn_prefill, for training through the
 * chunked form ("Inside Qwen3.5", section 5: the gated delta rule layer is
 * trained at scale; "Hybrid Mamba-Transformer MoE", the training
 * infrastructure section: the linear-recurrence layers need training paths
 * of their own).
 *
 * Given the forward call's inputs and the gradients of a loss with respect to
 * its outputs (d_o, d_final_state), writes the gradients with respect to q,
 * k, v (before the in-call L2 norm when GDN_FLAG_L2NORM_QK is set), g, beta
 * and the initial state.  It is reverse-mode differentiation of the same
 * recurrence: per chunk the state-independent quantities are recomputed, the
 * chunk-start states are rebuilt by a forward chain over the chunks, the
 * state gradients run back over the chunks, and each chunk's own gradients
 * follow from both.  Arithmetic is fp32 (bf16 inputs are widened exactly),
 * except that with bf16 inputs the two serial chains take bf16 MFMA
 * operands, as the forward scan does; their accumulators stay fp32.
 *
 *   flags, io_dtype, n_seqs, total_tokens, h_qk, h_v, d_k, d_v, chunk,
 *   scale, q, k, v (with their strides), g, beta, initial_state, cu_seqlens:
 *                exactly as passed to the forward gdn_prefill call.
 *                chunk in {16, 32, 64}: the gradients do not depend on it
 *                beyond rounding.
 *   d_o          [T, h_v, d_v] in io_dtype, contiguous.
 *   d_final_state [n_seqs, h_v, d_v, d_k] fp32, or NULL for zero.
 *   dq, dk       [T, h_qk, d_k] in io_dtype with token strides dq_stride and
 *                dk_stride; dv [T, h_v, d_v] with dv_stride (every token
 *                stride, inputs' included, a multiple of 8 elements).  They may be
 *                column slices of one [T, C] buffer (the conv output's
 *                gradient) and must not overlap any input.
 *   dg, dbeta    [T, h_v] fp32.
 *   d_initial_state [n_seqs, h_v, d_v, d_k] fp32, or NULL (not formed).
 *   workspace    at least gdn_prefill_backward_workspace_size() bytes,
 *                256-byte aligned; contents on entry are ignored.  It holds
 *                every chunk's intermediates, except when that would pass
 *                4 GiB.  Then one sequence (n_seqs = 1) runs in windows of
 *                whole chunks (a forward pass for the window-start states,
 *                then each window's backward, last to first), and the
 *                workspace holds one window plus the window-start states;
 *                a pack (n_seqs > 1) runs its sequences one after another,
 *                each as one sequence, in a workspace of 4 GiB or of one
 *                sequence holding every token, whichever is larger.  Such a
 *                pack call first copies cu_seqlens to the host, which
 *                synchronises the stream once; under stream capture it
 *                returns GDN_ERR_HIP (capture unsupported) before any launch.
 * Errors as gdn_prefill; every output is written in full on success.
 * ---------------------------------------------------------------------- */
typedef struct gdn_prefill_backward_args {
  uint32_t struct_size;
  uint32_t flags;
  int32_t io_dtype;
  int32_t n_seqs;
  int64_t total_tokens;
  int32_t h_qk;
  int32_t h_v;
  int32_t d_k;
  int32_t d_v;
  int32_t chunk;
  float scale;
  const void* q;
  const void* k;
  const void* v;
  int64_t q_stride;
  int64_t k_stride;
  int64_t v_stride;
  const float* g;
  const float* beta;
  const float* initial_state;
  const int32_t* cu_seqlens;
  const void* d_o;
  const float* d_final_state;
  void* dq;
  void* dk;
  void* dv;
  int64_t dq_stride;
  int64_t dk_stride;
  int64_t dv_stride;
  float* dg;
  float* dbeta;
  float* d_initial_state;
  void* workspace;
  size_t workspace_bytes;
} gdn_prefill_backward_args;

/* Bytes of workspace gdn_prefill_backward needs (pointers are not read);
 * 0 when the arguments are invalid. */
size_t gdn_prefill_backward_workspace_size(const gdn_prefill_backward_args* args);

gdn_status gdn_prefill_backward(const gdn_prefill_backward_args* args, void* stream);

/* ------------------------------------------------------------------------
 * gdn_conv1d_backward -- gradients of gdn_conv1d (same definition, "Inside
 * Qwen3.5", section 5, and the conv state of "Mamba hybrid model selection",
 * per-request memory section).
 *
 *   dtype, n_seqs, total_tokens, channels (multiple of 8), width,
 *   activation, x, weight, bias, cu_seqlens: as passed to the forward call
 *   (x 16-byte aligned).
 *   conv_state   [n_seqs, C, W-1] in dtype: the state the forward call READ
 *                (the forward overwrites its buffer, so keep a copy), or NULL
 *                for zeros.
 *   dy           [T, C] in dtype, 16-byte aligned: gradient of the loss with
 *                respect to y.
 *   d_new_state  [n_seqs, C, W-1] fp32 gradient with respect to the state the
 *                forward call wrote, or NULL for zero.
 *   dx           [T, C] in dtype, 16-byte aligned; must not overlap any
 *                input.
 *   dweight      [C, W] fp32;  dbias [C] fp32 or NULL (only with bias).
 *   d_conv_state [n_seqs, C, W-1] fp32, or NULL (not formed).
 *   workspace    at least gdn_conv1d_backward_workspace_size() bytes,
 *                256-byte aligned (partial weight sums over token tiles,
 *                added in a fixed order, so results are deterministic).
 * ---------------------------------------------------------------------- */
typedef struct gdn_conv1d_backward_args {
  uint32_t struct_size;
  int32_t dtype;
  int32_t n_seqs;
  int32_t channels;
  int64_t total_tokens;
  int32_t width;
  int32_t activation;
  const void* x;
  const void* weight;
  const void* bias;
  const void* conv_state;
  const int32_t* cu_seqlens;
  const void* dy;
  const float* d_new_state;
  void* dx;
  float* dweight;
  float* dbias;
  float* d_conv_state;
  void* workspace;
  size_t workspace_bytes;
} gdn_conv1d_backward_args;

size_t gdn_conv1d_backward_workspace_size(const gdn_conv1d_backward_args* args);

gdn_status gdn_conv1d_backward(const gdn_conv1d_backward_args* args, void* stream);

/* Diagnostics. */
const char* gdn_status_string(gdn_status status);
const char* gdn_last_error(void); /* thread-local detail of the last failure */
int gdn_abi_version(void);

/* Measurement aids: ceilings measured on the machine at hand, against which
 * a kernel's roofline fraction is also quoted.
 *   gdn_probe_mfma   launches `blocks` workgroups of four waves, each wave
 *                    issuing iters x 8 independent bf16 MFMAs (16x16x32);
 *                    writes one value per thread to out [blocks * 256] fp32
 *                    (device).  gdn_probe_mfma_flops gives the FLOPs of one
 *                    launch.
 *   gdn_probe_copy   copies `bytes` (a multiple of 16; 16-byte aligned,
 *                    non-overlapping device buffers) with streaming 16-byte
 *                    loads and stores.
 * Both return GDN_ERR_INVALID_ARG on bad arguments, GDN_ERR_HIP when the
 * launch fails. */
int64_t gdn_probe_mfma_flops(int32_t iters, int32_t blocks);
gdn_status gdn_probe_mfma(int32_t iters, int32_t blocks, float* out, void* stream);
gdn_status gdn_probe_copy(const void* src, void* dst, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
