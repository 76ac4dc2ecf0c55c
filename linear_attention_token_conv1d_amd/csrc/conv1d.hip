// gdn_conv1d: causal depthwise convolution (+ SiLU) over packed sequences.
//
// Main kernel: a workgroup covers 2048 channels (8 per thread, one 16-byte
// bf16 vector) by kTile consecutive tokens of the packed array.  Each thread
// walks its tokens in order keeping the last W-1 inputs of its 8 channels in
// registers, so every input is read once from HBM (plus a W-1 token halo per
// tile) and every output written once.  x loads for kBatch tokens are
// issued together before their use.  Sequence starts inside a tile reset the window
// from that sequence's conv state (or zeros), so nothing leaks across
// sequences.
//
// State kernel (launched after, on the same stream, so the main kernel has
// read every old state first): for each sequence, the new conv state is the
// last W-1 inputs of (old state ++ sequence), oldest first.
//
// Ring heads: with conv_head, input j (oldest first) of a stored state sits
// in slot (head + j) mod (W-1).  Both kernels read in that order; the state
// kernel writes chronologically and sets the head to 0.  Every state-kernel
// workgroup of a sequence reads its head, so the reset must wait until all
// of them have: each adds 1 << 8 to the head word when it reads it (the low
// 8 bits, the head, are unchanged), and the workgroup that finds the count
// of the others already there is the last reader and stores 0.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 16;   // tokens per workgroup (many workgroups keep more loads in flight)
constexpr int kBatch = 4;   // tokens whose loads are issued together

template <typename T> struct Vec8;
template <> struct Vec8<__bf16> { using type = uint4; };
template <> struct Vec8<float> { struct type { float4 a, b; }; };

template <typename T>
__device__ __forceinline__ typename Vec8<T>::type ld8raw(const T* p) {
  return *reinterpret_cast<const typename Vec8<T>::type*>(p);
}
__device__ __forceinline__ void unpack8(const uint4& w, float (&v)[8]) {
  v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x); v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
  v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z); v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
}
__device__ __forceinline__ void unpack8(const Vec8<float>::type& w, float (&v)[8]) {
  v[0] = w.a.x; v[1] = w.a.y; v[2] = w.a.z; v[3] = w.a.w;
  v[4] = w.b.x; v[5] = w.b.y; v[6] = w.b.z; v[7] = w.b.w;
}

// Largest s with cu[s] <= t (skipping empty sequences ending at t).
__device__ __forceinline__ int find_seq(const int32_t* cu, int n_seqs, int64_t t) {
  int lo = 0, hi = n_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((int64_t)cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// ring head of sequence s (0 without heads), reduced to a slot index
template <int W>
__device__ __forceinline__ int ring_head(const ConvParams& p, int s) {
  return p.conv_head ? (int)((uint32_t)(p.conv_head[s] & 0xff) % (W - 1)) : 0;
}

template <typename T, int W>
__device__ __forceinline__ void load_history(const ConvParams& p, int s, int64_t c0,
                                             float (&win)[W - 1][8]) {
  // positions before a sequence start: the conv state, oldest first, or zeros
  if (p.conv_state) {
    const T* st = reinterpret_cast<const T*>(p.conv_state) + ((int64_t)s * p.channels + c0) * (W - 1);
    const int h = ring_head<W>(p, s);
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int j = 0; j < W - 1; ++j) {
        const int slot = j + h < W - 1 ? j + h : j + h - (W - 1);
        win[j][e] = to_f32(st[e * (W - 1) + slot]);
      }
  } else {
#pragma unroll
    for (int j = 0; j < W - 1; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) win[j][e] = 0.f;
  }
}

template <typename T, int W>
__global__ __launch_bounds__(kThreads) void conv1d_kernel(ConvParams p) {
  const int64_t c0 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * 8;
  if (c0 >= p.channels) return;
  const int64_t C = p.channels;
  const int64_t t0 = (int64_t)blockIdx.y * kTile;
  const int64_t t1 = min(t0 + (int64_t)kTile, p.total_tokens);
  const T* x = reinterpret_cast<const T*>(p.x);
  T* y = reinterpret_cast<T*>(p.y);

  int s = 0;
  int64_t seq_start = 0, seq_end = p.total_tokens;
  if (p.cu_seqlens) {
    s = find_seq(p.cu_seqlens, p.n_seqs, t0);
    seq_start = p.cu_seqlens[s];
    seq_end = p.cu_seqlens[s + 1];
  }

  float w[W][8];
  {
    const T* wp = reinterpret_cast<const T*>(p.weight) + c0 * W;
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int j = 0; j < W; ++j) w[j][e] = to_f32(wp[e * W + j]);
  }
  float bias[8];
#pragma unroll
  for (int e = 0; e < 8; ++e)
    bias[e] = p.bias ? to_f32(reinterpret_cast<const T*>(p.bias)[c0 + e]) : 0.f;

  // window: win[W-2] is the most recent input before the current token.
  // Positions before the sequence start come from its conv state: position
  // seq_start - m sits in state slot (W-1) - m.
  float win[W - 1][8];
  {
    float hist[W - 1][8];
    load_history<T, W>(p, s, c0, hist);
#pragma unroll
    for (int m = 1; m < W; ++m) {
      const int64_t pos = t0 - m;
      if (pos >= seq_start) {
        float v[8];
        unpack8(ld8raw(x + pos * C + c0), v);
#pragma unroll
        for (int e = 0; e < 8; ++e) win[W - 1 - m][e] = v[e];
      } else {
        const int64_t back = seq_start - pos;  // 1 .. W-1
#pragma unroll
        for (int j = 0; j < W - 1; ++j)
          if (j == (W - 1) - back)
#pragma unroll
            for (int e = 0; e < 8; ++e) win[W - 1 - m][e] = hist[j][e];
      }
    }
  }

  // fast path: a full tile inside one sequence.  Every load of a batch is
  // issued with no branch around it, so the batch's loads are in flight
  // together.
  if (t1 - t0 == kTile && seq_end >= t1) {
    for (int64_t tb = t0; tb < t1; tb += kBatch) {
      typename Vec8<T>::type raw[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) raw[i] = ld8raw(x + (tb + i) * C + c0);
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        float xv[8];
        unpack8(raw[i], xv);
        float out[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float acc = bias[e];
#pragma unroll
          for (int j = 0; j < W - 1; ++j) acc += w[j][e] * win[j][e];
          acc += w[W - 1][e] * xv[e];
          out[e] = p.act ? silu(acc) : acc;
        }
        store8(y + (tb + i) * C + c0, out);
#pragma unroll
        for (int j = 0; j + 1 < W - 1; ++j)
#pragma unroll
          for (int e = 0; e < 8; ++e) win[j][e] = win[j + 1][e];
#pragma unroll
        for (int e = 0; e < 8; ++e) win[W - 2][e] = xv[e];
      }
    }
    return;
  }
  for (int64_t tb = t0; tb < t1; tb += kBatch) {
    typename Vec8<T>::type raw[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i)
      if (tb + i < t1) raw[i] = ld8raw(x + (tb + i) * C + c0);
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int64_t t = tb + i;
      if (t < t1) {
        if (t == seq_end) {  // a new sequence starts here (skip empty ones)
          do { ++s; seq_end = p.cu_seqlens[s + 1]; } while (seq_end == t);
          load_history<T, W>(p, s, c0, win);
        }
        float xv[8];
        unpack8(raw[i], xv);
        float out[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float acc = bias[e];
#pragma unroll
          for (int j = 0; j < W - 1; ++j) acc += w[j][e] * win[j][e];
          acc += w[W - 1][e] * xv[e];
          out[e] = p.act ? silu(acc) : acc;
        }
        store8(y + t * C + c0, out);
#pragma unroll
        for (int j = 0; j + 1 < W - 1; ++j)
#pragma unroll
          for (int e = 0; e < 8; ++e) win[j][e] = win[j + 1][e];
#pragma unroll
        for (int e = 0; e < 8; ++e) win[W - 2][e] = xv[e];
      }
    }
  }
}

// Ring heads of a chronological rewrite: every workgroup of sequence s reads
// its head once; after all of its threads have, thread 0 counts the
// workgroup in, and the last of the sequence's workgroups stores head 0.
__device__ __forceinline__ void release_head(const ConvParams& p, int s) {
  if (!p.conv_head) return;
  __syncthreads();  // every thread of this workgroup has used the head
  if (threadIdx.x == 0) {
    const int readers = (int)gridDim.x;
    const int32_t before = atomicAdd(p.conv_head + s, 1 << 8);
    if ((before >> 8) == readers - 1) atomicExch(p.conv_head + s, 0);
  }
}

template <typename T, int W>
__global__ __launch_bounds__(kThreads) void conv_state_kernel(ConvParams p) {
  const int64_t c0 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * 8;
  const int s = blockIdx.y;
  if (c0 < p.channels) {
    const int64_t C = p.channels;
    const int64_t start = p.cu_seqlens ? p.cu_seqlens[s] : 0;
    const int64_t end = p.cu_seqlens ? p.cu_seqlens[s + 1] : p.total_tokens;
    const T* x = reinterpret_cast<const T*>(p.x);
    T* st = reinterpret_cast<T*>(p.conv_state) + ((int64_t)s * C + c0) * (W - 1);
    // old state, oldest first (ring order with a head)
    const int h = ring_head<W>(p, s);
    float old[W - 1][8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int j = 0; j < W - 1; ++j) {
        const int slot = j + h < W - 1 ? j + h : j + h - (W - 1);
        old[j][e] = to_f32(st[e * (W - 1) + slot]);
      }
    float nw[W - 1][8];
#pragma unroll
    for (int j = 0; j < W - 1; ++j) {
      const int64_t pos = end - (W - 1) + j;  // position of new slot j
      if (pos >= start) {
        float v[8];
        unpack8(ld8raw(x + pos * C + c0), v);
#pragma unroll
        for (int e = 0; e < 8; ++e) nw[j][e] = v[e];
      } else {
        const int64_t back = (W - 1) - (start - pos);  // still inside the old state
#pragma unroll
        for (int i = 0; i < W - 1; ++i)
          if (i == back)
#pragma unroll
            for (int e = 0; e < 8; ++e) nw[j][e] = old[i][e];
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int j = 0; j < W - 1; ++j) st[e * (W - 1) + j] = from_f32<T>(nw[j][e]);
  }
  release_head(p, s);
}

template <typename T, int W>
hipError_t launch_t(const ConvParams& p, hipStream_t stream) {
  const unsigned cblocks = (unsigned)((p.channels / 8 + kThreads - 1) / kThreads);
  if (p.total_tokens > 0) {
    const unsigned tiles = (unsigned)((p.total_tokens + kTile - 1) / kTile);
    hipLaunchKernelGGL((conv1d_kernel<T, W>), dim3(cblocks, tiles), dim3(kThreads), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.conv_state) {
    hipLaunchKernelGGL((conv_state_kernel<T, W>), dim3(cblocks, (unsigned)p.n_seqs), dim3(kThreads),
                       0, stream, p);
    return hipGetLastError();
  }
  return hipSuccess;
}

template <typename T>
hipError_t launch_w(const ConvParams& p, hipStream_t stream) {
  switch (p.width) {
    case 2: return launch_t<T, 2>(p, stream);
    case 3: return launch_t<T, 3>(p, stream);
    default: return launch_t<T, 4>(p, stream);
  }
}

}  // namespace

hipError_t launch_conv1d(const ConvParams& p, int dtype, hipStream_t stream) {
  return dtype == 1 ? launch_w<__bf16>(p, stream) : launch_w<float>(p, stream);
}

}  // namespace gdn
