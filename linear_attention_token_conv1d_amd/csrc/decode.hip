// gdn_decode_step kernel: one token for each of N sequences.
//
// One workgroup owns (sequence n, QK head hq) and therefore the grp = h_v/h_qk
// V heads that read that QK head.  It
//   1. runs the conv step (+ SiLU) for its q, k and v channels, storing the
//      new input in the conv state (each channel is read and written by the
//      thread that owns it, so the in-place update is race-free): without
//      ring heads the W-1 slots shift; with them only slot `head` (the
//      oldest input) is overwritten, and the last of the sequence's h_qk
//      workgroups to read the head advances it (each adds 1 << 8 to the head
//      word after reading it, keeping the low 8 bits, so the one that finds
//      the other h_qk - 1 counts there knows every reader is done);
//   2. L2-normalises q and k (one wave, fp32);
//   3. streams the grp*d_v state rows once: each row S_i (d_k values) is
//      loaded by 16 lanes, reduced against k and q with DPP row sums, then
//        a_i = S_i.k,  b_i = S_i.q,  d_i = beta (v_i - alpha a_i)  (beta v_i
//        without the erase)
//        S_i <- alpha S_i + d_i k^T,  o_i = scale (alpha b_i + d_i (k.q))
//      and written back.  Rows are independent, so one pass suffices: the
//      kernel reads and writes each state byte exactly once.
// The state of a workgroup (grp*d_v rows of d_k) is contiguous in memory, so a
// wave moves 4 consecutive rows (1 KiB of bf16) per 16-byte-per-lane access.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
#ifndef GDN_DECODE_UNROLL
#define GDN_DECODE_UNROLL 8
#endif
// row groups of 16 rows whose loads a wave keeps in flight together
constexpr int kConvBatch = 4;  // conv channels per thread whose loads issue together
template <int D>
constexpr int kUnroll = GDN_DECODE_UNROLL * 16 <= D ? GDN_DECODE_UNROLL : D / 16;

// State rows are read and written once per step: streaming accesses.  A
// row is PE-element pieces (16 bytes, or the lane's whole share when that is
// less), and the 16 lanes of a row take consecutive pieces: lane sub holds
// pieces j * 16 + sub (j < EPL / PE), so every load and store instruction
// covers one contiguous span.  Element e of the lane is d_k index
// elem_d(sub, e).
template <typename T, int EPL>
constexpr int kPE = 16 / (int)sizeof(T) < EPL ? 16 / (int)sizeof(T) : EPL;
template <typename T, int EPL>
__device__ __forceinline__ int elem_d(int sub, int e) {
  constexpr int PE = kPE<T, EPL>;
  return ((e / PE) * 16 + sub) * PE + e % PE;
}
template <int EPL, typename T>
__device__ __forceinline__ void load_row(const T* row, int sub, float (&v)[EPL]) {
  constexpr int PE = kPE<T, EPL>;
  static_assert(PE == 8 || PE == 4, "8- or 4-element pieces");
#pragma unroll
  for (int j = 0; j < EPL / PE; ++j) {
    float w[PE];
    if constexpr (PE == 8) load8_stream(row + (j * 16 + sub) * PE, w); else load4_stream(row + (j * 16 + sub) * PE, w);
#pragma unroll
    for (int i = 0; i < PE; ++i) v[j * PE + i] = w[i];
  }
}
template <int EPL, typename T>
__device__ __forceinline__ void store_row(T* row, int sub, const float (&v)[EPL]) {
  constexpr int PE = kPE<T, EPL>;
#pragma unroll
  for (int j = 0; j < EPL / PE; ++j) {
    float w[PE];
#pragma unroll
    for (int i = 0; i < PE; ++i) w[i] = v[j * PE + i];
    if constexpr (PE == 8) store8_stream(row + (j * 16 + sub) * PE, w); else store4_stream(row + (j * 16 + sub) * PE, w);
  }
}

template <typename IoT, typename StT, int D>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeParams p) {
  constexpr int EPL = D / 16;  // state elements per lane per row
  extern __shared__ float smem[];
  const int grp = p.h_v / p.h_qk;
  const int n = blockIdx.x / p.h_qk;
  const int hq = blockIdx.x - n * p.h_qk;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  float* s_q = smem;               // [D]        q, then k, then v: channel order
  float* s_k = s_q + D;            // [D]
  float* s_v = s_k + D;            // [grp*D]
  float* s_o = s_v + grp * D;      // [grp*D]
  float* s_al = s_o + grp * D;     // [grp] alpha
  float* s_be = s_al + grp;        // [grp] beta
  float* s_sc = s_be + grp;        // rq, rk, k.q

  // The state stream does not depend on the conv step: the first pass of
  // state loads is issued now so that its latency overlaps steps 1 and 2.
  // A pass covers 16 * U consecutive rows, which divides rows = grp * D:
  // every row group of a pass exists, so its loads issue back to back with
  // no branch between them.
  constexpr int U = kUnroll<D>;
  static_assert(D % (16 * U) == 0, "rows per pass must divide grp * D");
  static_assert(U % 2 == 0, "a pass is streamed in two halves");
  const int rows = grp * D;
  const int sub = lane & 15;
  // state and conv-state slot of sequence n
  const int64_t slot = p.state_idx ? as_const(p.state_idx)[n] : n;
  StT* S = reinterpret_cast<StT*>(p.state) + (slot * p.h_v + (int64_t)hq * grp) * D * D;
  int rb = wave * 4 + (lane >> 4);
  float sv[U][EPL];
#pragma unroll
  for (int u = 0; u < U; ++u) load_row<EPL>(S + (int64_t)(rb + 16 * u) * D, sub, sv[u]);

  // ---- 1. conv step + activation over this workgroup's channels.  A thread
  // handles up to kConvBatch channels at a time and issues every load of the
  // batch (input, taps, history, bias) before using any of them; out-of-range
  // slots and taps load a clamped, valid address and are discarded.
  const int64_t C = (int64_t)(2 * p.h_qk + p.h_v) * D;
  const IoT* x = reinterpret_cast<const IoT*>(p.x) + (int64_t)n * C;
  const int nloc = (2 + grp) * D;
  const int W = p.width;  // 2..4
  const int64_t gi = (int64_t)n * p.h_v + (int64_t)hq * grp + min(tid, grp - 1);
  const float g_in = p.g[gi], b_in = p.beta[gi];  // stored to LDS after the conv loads
  const IoT* wt = reinterpret_cast<const IoT*>(p.conv_weight);
  const IoT* bias = reinterpret_cast<const IoT*>(p.conv_bias);
  IoT* cst = reinterpret_cast<IoT*>(p.conv_state);
  // ring head of this sequence's conv state (0 and a shift without heads)
  const bool ring = p.conv_head != nullptr;
  const int head = ring ? (int)((uint32_t)(p.conv_head[slot] & 0xff) % (uint32_t)(W - 1)) : 0;
  auto conv_batch = [&](int base) {
    int64_t cc[kConvBatch];
    IoT xr[kConvBatch], wv[kConvBatch][4], hv[kConvBatch][3], bv[kConvBatch];
#pragma unroll
    for (int j = 0; j < kConvBatch; ++j) {
      const int cl = min(base + j * kThreads + tid, nloc - 1);
      int64_t c;
      if (cl < D) c = (int64_t)hq * D + cl;
      else if (cl < 2 * D) c = (int64_t)(p.h_qk + hq) * D + (cl - D);
      else c = (int64_t)2 * p.h_qk * D + (int64_t)hq * grp * D + (cl - 2 * D);
      cc[j] = c;
      xr[j] = x[c];
      // without a conv (or a bias) the loads read x[c] instead and are unused:
      // no branch separates the loads of a batch
      const IoT* wp = wt ? wt + c * W : x + c;
      const IoT* st = wt ? cst + (slot * C + c) * (W - 1) : x + c;
      const int wm = wt ? W - 1 : 0, hm = wt ? W - 2 : 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) wv[j][i] = wp[min(i, wm)];
      // history i (oldest first) sits in slot (head + i) mod (W - 1)
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        const int hi = min(i, hm) + head;
        hv[j][i] = st[hi < W - 1 ? hi : hi - (W - 1)];
      }
      bv[j] = bias ? bias[c] : x[c];
    }
#pragma unroll
    for (int j = 0; j < kConvBatch; ++j) {
      const int cl = base + j * kThreads + tid;
      if (cl >= nloc) continue;
      float y = to_f32(xr[j]);
      if (wt) {
        // taps 0..W-2 meet the history (oldest first), tap W-1 the new input
        float acc = bias ? to_f32(bv[j]) : 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float xi = i < W - 1 ? to_f32(hv[j][min(i, 2)]) : (i == W - 1 ? y : 0.f);
          acc += to_f32(wv[j][i]) * xi;
        }
        // the history keeps the last W-1 inputs: the new one replaces the
        // oldest (ring), or everything shifts by one slot
        IoT* st = cst + (slot * C + cc[j]) * (W - 1);
        if (ring) {
          st[head] = xr[j];
        } else {
#pragma unroll
          for (int i = 0; i < 3; ++i)
            if (i < W - 1) st[i] = i + 1 < W - 1 ? hv[j][min(i + 1, 2)] : xr[j];
        }
        y = p.act ? silu(acc) : acc;
      }
      s_q[cl] = y;
    }
  };
  // the first batch is peeled off the loop: inside a loop the compiler's wait
  // counts merge with the previous iteration and would stall on the state
  // loads issued above
  conv_batch(0);
  for (int base = kConvBatch * kThreads; base < nloc; base += kConvBatch * kThreads) conv_batch(base);
  if (tid < grp) {
    s_al[tid] = __expf(g_in);
    s_be[tid] = b_in;
  }
  __syncthreads();
  // every thread of this workgroup has read the ring head: count the
  // workgroup in; the sequence's last reader advances the head
  if (ring && tid == 0) {
    const int32_t before = atomicAdd(p.conv_head + slot, 1 << 8);
    if ((before >> 8) == p.h_qk - 1) atomicExch(p.conv_head + slot, (int32_t)((head + 1) % (W - 1)));
  }

  // ---- 2. L2 norms of q and k, and k.q after normalisation
  if (wave == 0) {
    float sq = 0.f, sk = 0.f, sqk = 0.f;
    for (int i = lane; i < D; i += 64) {
      const float a = s_q[i], b = s_k[i];
      sq += a * a; sk += b * b; sqk += a * b;
    }
    sq = wave_sum(sq); sk = wave_sum(sk); sqk = wave_sum(sqk);
    if (lane == 0) {
      const float rq = p.l2norm ? 1.0f / sqrtf(sq + 1e-6f) : 1.0f;
      const float rk = p.l2norm ? 1.0f / sqrtf(sk + 1e-6f) : 1.0f;
      s_sc[0] = rq; s_sc[1] = rk; s_sc[2] = sqk * rq * rk;
    }
  }
  __syncthreads();

  // ---- 3. stream the state rows once
  const float rq = s_sc[0], rk = s_sc[1], kq = s_sc[2];
  float kf[EPL], qf[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    kf[e] = s_k[elem_d<StT, EPL>(sub, e)] * rk;
    qf[e] = s_q[elem_d<StT, EPL>(sub, e)] * rq;
  }
  auto row_step = [&](int u) {
    const int r = rb + 16 * u;
    float a = 0.f, b = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) { a += sv[u][e] * kf[e]; b += sv[u][e] * qf[e]; }
    a = row16_sum(a);
    b = row16_sum(b);
    const int hl = r / D;
    const float al = s_al[hl];
    const float dl = s_be[hl] * (s_v[r] - (p.erase ? al * a : 0.f));
    float nv[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) nv[e] = al * sv[u][e] + dl * kf[e];
    store_row<EPL>(S + (int64_t)r * D, sub, nv);
    if (sub == 0) s_o[r] = p.scale * (al * b + dl * kq);
  };
  // The row groups of a pass are processed in two halves; once a half is
  // written back its registers load the same half of the next pass, so loads
  // stay in flight while the other half is computed.  The last pass has its
  // own copy of the second half, which keeps every load outside a branch.
  constexpr int H = U / 2;
  while (true) {
#pragma unroll
    for (int u = 0; u < H; ++u) row_step(u);
    if (rb + 16 * U >= rows) {
#pragma unroll
      for (int u = H; u < U; ++u) row_step(u);
      break;
    }
#pragma unroll
    for (int u = 0; u < H; ++u) load_row<EPL>(S + (int64_t)(rb + 16 * U + 16 * u) * D, sub, sv[u]);
#pragma unroll
    for (int u = H; u < U; ++u) row_step(u);
#pragma unroll
    for (int u = H; u < U; ++u) load_row<EPL>(S + (int64_t)(rb + 16 * U + 16 * u) * D, sub, sv[u]);
    rb += 16 * U;
  }
  __syncthreads();
  IoT* o = reinterpret_cast<IoT*>(p.o) + ((int64_t)n * p.h_v + (int64_t)hq * grp) * D;
  for (int i = tid; i < rows; i += kThreads) o[i] = from_f32<IoT>(s_o[i]);
}

template <typename IoT, typename StT, int D>
hipError_t launch_t(const DecodeParams& p, hipStream_t stream) {
  const int grp = p.h_v / p.h_qk;
  const size_t shmem = sizeof(float) * ((size_t)(2 + 2 * grp) * D + 2 * grp + 4);
  const unsigned blocks = (unsigned)((int64_t)p.n_seqs * p.h_qk);
  hipLaunchKernelGGL((decode_kernel<IoT, StT, D>), dim3(blocks), dim3(kThreads), shmem, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int io_dtype, int state_dtype, int d,
                         hipStream_t stream) {
  const bool io_bf = io_dtype == 1, st_bf = state_dtype == 1;
  if (d == 128) {
    if (io_bf) return st_bf ? launch_t<__bf16, __bf16, 128>(p, stream) : launch_t<__bf16, float, 128>(p, stream);
    return st_bf ? launch_t<float, __bf16, 128>(p, stream) : launch_t<float, float, 128>(p, stream);
  }
  if (io_bf) return st_bf ? launch_t<__bf16, __bf16, 64>(p, stream) : launch_t<__bf16, float, 64>(p, stream);
  return st_bf ? launch_t<float, __bf16, 64>(p, stream) : launch_t<float, float, 64>(p, stream);
}

}  // namespace gdn
