// Backward pass of the token mixer, for training: gradients of the chunked
// gated delta rule (gdn_prefill) and of the causal conv (gdn_conv1d).
//
// Per chunk of one sequence and one V head (K^, Q^ the normalised keys and
// queries, rows past the chunk's end padded with zeros and beta = g = 0, so
// every chunk is a full C rows), the forward is the recurrence of "Inside
// Qwen3.5", sections 4-5, unrolled over one chunk (an exact rearrangement):
//   G = cumsum(g), gam = e^G, e_j = e^{G_{C-1} - G_j}, Gam_rj = e^{G_r - G_j}
//   A = strict_lower(beta_r Gam_rj K^_r.K^_j),  T = (I + A)^-1
//   W = T diag(beta gam) K^,  Ut = T diag(beta) V,  U = Ut - W X
//   Pm = scale lower_incl(Gam o Q^K^T),  O = scale diag(gam) Q^ X + Pm U
//   X' = gam_{C-1} X + (diag(e) K^)^T U
// with X = S^T (d_k x d_v) the state at the chunk start.  The backward takes
// these steps back in the opposite order:
//   1. recompute everything that does not depend on the state (batched
//      products over (chunk, head));
//   2. rebuild the chunk-start states X_c by running the chain forward;
//   3. run the state gradient back over the chunks:
//        dU = Pm^T dO + diag(e) K^ dX',  dX = gam dX' + (scale diag(gam) Q^)^T dO - W^T dU
//   4. per chunk, the gradients of every chunk-local quantity, down to
//      dK^, dQ^, dV, dbeta and dG (then dg is the reverse cumulative sum of dG);
//   5. dK^ and dQ^ of a QK head add up over the V heads that read it and
//      pass back through the L2 norm.
// The stages: a batched fp32-MFMA GEMM over (chunk, head) for the
// state-independent products, one launch that runs both serial chains (bf16
// MFMA operands for bf16 inputs, fp32 VALU for fp32 inputs, fp32 state either
// way), one fused kernel per (chunk, V head) for every chunk-local gradient,
// and a per-token kernel for the QK-head sums and the L2-norm backward.
// Every array passed between stages is an fp32 workspace array.
#include <algorithm>
#include <cstdlib>
#include <type_traits>
#include <vector>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

// ------------------------------------------------------------- workspace
// Header: [0] number of chunks in use, then chunk offsets per sequence
// (n_seqs + 1), then one (sequence, first token, rows) record per chunk.
// Then fp32 arrays, each [max_chunks][heads][rows][cols]:
//   per QK head: Kn, Qn (C x D), KK, QK (C x C)
//   per V head:  vec (6 x C), two C x C, nine C x D and three D x D
// vec rows: G, gam, e, beta, beta gam (0 without the erase term) and scale
// gam; the last two scale K^ and Q^ rows on the fly
enum { kVecG = 0, kVecGam, kVecE, kVecBeta, kVecBG, kVecSG, kNVec };
enum { cT = 0, cPm, kNCC };
enum { mBV = 0, mDO, mW, mUt, mU, mDU, mPdO, mDKn, mDQn, kNCD };
enum { xXs = 0, xDXs, xZ, kNDD };

struct ChunkRec {
  int n, t0, len, pad;
};

struct BwdWs {
  int* nc;
  int* co;
  ChunkRec* ct;
  float *Kn, *Qn, *KK, *QK;
  float* vec;
  float* cc[kNCC];
  float* cd[kNCD];
  float* dd[kNDD];
};

__host__ __device__ inline size_t a256(size_t x) { return (x + 255) / 256 * 256; }

struct BwdSizes {
  int64_t ncm;
  size_t o_ct, hdr, total;
};

inline BwdSizes bwd_sizes(int64_t T, int n_seqs, int h_qk, int h_v, int D, int C) {
  BwdSizes s;
  s.ncm = T / C + n_seqs;
  s.o_ct = (4 * (4 + (size_t)n_seqs + 1) + 15) / 16 * 16;
  s.hdr = a256(s.o_ct + sizeof(ChunkRec) * (size_t)s.ncm);
  const size_t cq = (size_t)s.ncm * h_qk, cv = (size_t)s.ncm * h_v;
  size_t f = 0;
  f += a256(cq * C * D * 4) * 2 + a256(cq * C * C * 4) * 2;
  f += a256(cv * kNVec * C * 4);
  f += a256(cv * C * C * 4) * kNCC;
  f += a256(cv * C * D * 4) * kNCD;
  f += a256(cv * D * D * 4) * kNDD;
  s.total = s.hdr + f;
  return s;
}

inline BwdWs bwd_carve(void* ws, int64_t T, int n_seqs, int h_qk, int h_v, int D, int C) {
  const BwdSizes s = bwd_sizes(T, n_seqs, h_qk, h_v, D, C);
  char* b = static_cast<char*>(ws);
  BwdWs w;
  w.nc = reinterpret_cast<int*>(b);
  w.co = w.nc + 4;
  w.ct = reinterpret_cast<ChunkRec*>(b + s.o_ct);
  size_t o = s.hdr;
  const size_t cq = (size_t)s.ncm * h_qk, cv = (size_t)s.ncm * h_v;
  auto take = [&](size_t bytes) {
    float* p = reinterpret_cast<float*>(b + o);
    o += a256(bytes);
    return p;
  };
  w.Kn = take(cq * C * D * 4);
  w.Qn = take(cq * C * D * 4);
  w.KK = take(cq * C * C * 4);
  w.QK = take(cq * C * C * 4);
  w.vec = take(cv * kNVec * C * 4);
  for (int i = 0; i < kNCC; ++i) w.cc[i] = take(cv * C * C * 4);
  for (int i = 0; i < kNCD; ++i) w.cd[i] = take(cv * C * D * 4);
  for (int i = 0; i < kNDD; ++i) w.dd[i] = take(cv * D * D * 4);
  return w;
}

// Sequence of packed token t: the last n with cu[n] <= t (which skips empty
// sequences that start at t, and has cu[n + 1] > t since t < cu[n_seqs]).
__device__ inline int seq_index(const int32_t* cu, int n_seqs, int64_t t) {
  int lo = 0, hi = n_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (cu[mid] <= t) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// ------------------------------------------------------------------ plan
// One workgroup: chunk offsets of every sequence (exclusive prefix sum of
// ceil(len / C)), then one record per chunk.
__global__ __launch_bounds__(256) void bwd_plan_kernel(BwdWs w, const int32_t* cu, int n_seqs, int64_t T,
                                                       int C, int64_t ncm) {
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int n = 0; n < n_seqs; ++n) {
      w.co[n] = acc;
      const int len = cu ? cu[n + 1] - cu[n] : (int)T;
      acc += (len + C - 1) / C;
    }
    w.co[n_seqs] = acc;
    w.nc[0] = acc;
  }
  __syncthreads();
  for (int n = threadIdx.x; n < n_seqs; n += blockDim.x) {
    const int s = cu ? cu[n] : 0, len = cu ? cu[n + 1] - s : (int)T;
    for (int c = 0, gc = w.co[n]; c * C < len; ++c, ++gc) w.ct[gc] = ChunkRec{n, s + c * C, min(C, len - c * C), 0};
  }
  for (int64_t gc = w.co[n_seqs] + threadIdx.x; gc < ncm; gc += blockDim.x) w.ct[gc] = ChunkRec{0, 0, 0, 0};
}

// ---------------------------------------------------------- batched GEMM
// C[b] = alpha op(A[b]) op(B[b]) (+ C[b] when accum), fp32, for every chunk
// b = (chunk, head) in use; an operand may have each stored row scaled first.  op(A) is M x K (A row-major M x K, or K x M when
// ta), op(B) is K x N (B row-major K x N, or N x K when tb).  A QK-head
// operand is shared by the V heads of its group (head index / hdiv).
struct BG {
  const float* A;
  const float* B;
  float* Cm;
  int M, N, K, lda, ldb, ldc;
  int64_t a_sc, a_sh, b_sc, b_sh, c_sc, c_sh;
  int a_hdiv, b_hdiv, H, ta, tb, accum;
  float alpha;
  const int* nc;
  // optional per-row scales of the stored operand rows (a row of the per
  // (chunk, V head) vec block, e.g. beta gam for the rows of K^), or null
  const float* as;
  const float* bs;
  int vstr;  // floats per (chunk, head) vec block
};

typedef float v4f __attribute__((ext_vector_type(4)));

// Workgroup barrier that waits for this wave's LDS operations only (vector
// memory loads and stores stay in flight: the compiler still waits for a
// load before its value is used).  __syncthreads() would also drain every
// outstanding global access, a prefetch of the next stage included.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));  // vmcnt 63, expcnt 7, lgkmcnt 0
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// A 64 x 64 output tile per workgroup on fp32 MFMA (16x16x4): wave w owns the
// 32 x 32 quadrant (w / 2, w % 2) as four 16 x 16 accumulators.  K is staged
// 32 at a time through LDS (k-major, so both operands are read with
// consecutive lanes on consecutive rows / columns); the next stage's global
// loads are issued before the current stage's MFMAs.  In a 16x16x4 MFMA lane
// l supplies A[l % 16][l / 16] and B[l / 16][l % 16] of its 16 x 4 and
// 4 x 16 slices, and holds C rows 4 (l / 16) .. +3 of column l % 16.
constexpr int kGK = 32;
// Global -> registers for one 32-deep stage: two 16-byte loads per operand
// per thread (M, N and K are multiples of 16, so a 4-element group is
// either wholly inside or wholly outside the matrix).
__device__ __forceinline__ void bg_fetch(const BG& p, const float* A, const float* B, const float* as,
                                         const float* bs, int m0, int n0, int k0, int tid, v4f (&ra)[2],
                                         v4f (&rb)[2]) {
  const v4f z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int f = tid + 256 * u;
    int ar, br;  // stored rows of the two groups
    if (p.ta) {  // A stored [k][m]: 4 consecutive m
      const int k = k0 + (f >> 4), m = m0 + (f & 15) * 4;
      ar = k;
      ra[u] = (k < p.K && m < p.M) ? *reinterpret_cast<const v4f*>(A + (int64_t)k * p.lda + m) : z;
    } else {     // A stored [m][k]: 4 consecutive k
      const int m = m0 + (f >> 3), k = k0 + (f & 7) * 4;
      ar = m;
      ra[u] = (m < p.M && k < p.K) ? *reinterpret_cast<const v4f*>(A + (int64_t)m * p.lda + k) : z;
    }
    if (p.tb) {  // B stored [n][k]: 4 consecutive k
      const int n = n0 + (f >> 3), k = k0 + (f & 7) * 4;
      br = n;
      rb[u] = (n < p.N && k < p.K) ? *reinterpret_cast<const v4f*>(B + (int64_t)n * p.ldb + k) : z;
    } else {     // B stored [k][n]: 4 consecutive n
      const int k = k0 + (f >> 4), n = n0 + (f & 15) * 4;
      br = k;
      rb[u] = (k < p.K && n < p.N) ? *reinterpret_cast<const v4f*>(B + (int64_t)k * p.ldb + n) : z;
    }
    if (as && ar < (p.ta ? p.K : p.M)) ra[u] *= as[ar];
    if (bs && br < (p.tb ? p.N : p.K)) rb[u] *= bs[br];
  }
}

__global__ __launch_bounds__(256) void bgemm_kernel(BG p) {
  const int z = blockIdx.x, gc = z / p.H, h = z % p.H;
  if (gc >= *p.nc) return;
  const int tiles_n = (p.N + 63) / 64;
  const int m0 = (blockIdx.y / tiles_n) * 64, n0 = (blockIdx.y % tiles_n) * 64;
  const float* A = p.A + gc * p.a_sc + (int64_t)(h / p.a_hdiv) * p.a_sh;
  const float* B = p.B + gc * p.b_sc + (int64_t)(h / p.b_hdiv) * p.b_sh;
  float* Cm = p.Cm + gc * p.c_sc + (int64_t)h * p.c_sh;
  const int64_t vb = ((int64_t)gc * p.H + h) * p.vstr;  // vec block of this (chunk, head)
  const float* as = p.as ? p.as + vb : nullptr;
  const float* bs = p.bs ? p.bs + vb : nullptr;
  __shared__ float smem[2 * kGK * 68];  // A and B stages; the output tile at the end
  float(*As)[68] = reinterpret_cast<float(*)[68]>(smem);
  float(*Bs)[68] = reinterpret_cast<float(*)[68]>(smem + kGK * 68);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int mw = (wave >> 1) * 32, nw = (wave & 1) * 32, l16 = lane & 15, g4 = lane >> 4;
  v4f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  v4f ra[2], rb[2];
  bg_fetch(p, A, B, as, bs, m0, n0, 0, tid, ra, rb);
  for (int k0 = 0; k0 < p.K; k0 += kGK) {
    lds_barrier();  // the previous stage's MFMAs are done reading As, Bs
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int f = tid + 256 * u;
      if (p.ta) {
        *reinterpret_cast<v4f*>(&As[f >> 4][(f & 15) * 4]) = ra[u];
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) As[(f & 7) * 4 + j][f >> 3] = ra[u][j];
      }
      if (p.tb) {
#pragma unroll
        for (int j = 0; j < 4; ++j) Bs[(f & 7) * 4 + j][f >> 3] = rb[u][j];
      } else {
        *reinterpret_cast<v4f*>(&Bs[f >> 4][(f & 15) * 4]) = rb[u];
      }
    }
    if (k0 + kGK < p.K) bg_fetch(p, A, B, as, bs, m0, n0, k0 + kGK, tid, ra, rb);
    lds_barrier();
#pragma unroll
    for (int ks = 0; ks < kGK; ks += 4) {
      const float a0 = As[ks + g4][mw + l16], a1 = As[ks + g4][mw + 16 + l16];
      const float b0 = Bs[ks + g4][nw + l16], b1 = Bs[ks + g4][nw + 16 + l16];
      acc[0][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, b0, acc[0][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, b1, acc[0][1], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, b0, acc[1][0], 0, 0, 0);
      acc[1][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, b1, acc[1][1], 0, 0, 0);
    }
  }
  // the 64 x 64 tile through LDS, then whole 16-byte rows to memory
  float(*Cs)[68] = reinterpret_cast<float(*)[68]>(smem);
  lds_barrier();
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) Cs[mw + 16 * i + 4 * g4 + r][nw + 16 * j + l16] = p.alpha * acc[i][j][r];
  lds_barrier();
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int f = tid + 256 * u, mm = f >> 4, n4 = (f & 15) * 4;
    const int m = m0 + mm, n = n0 + n4;
    if (m < p.M && n < p.N) {
      v4f* c = reinterpret_cast<v4f*>(Cm + (int64_t)m * p.ldc + n);
      v4f v = *reinterpret_cast<const v4f*>(&Cs[mm][n4]);
      if (p.accum) v += *c;
      *c = v;
    }
  }
}

// ------------------------------------------------------- stage: Kn, Qn
// Two consecutive elements (4-byte aligned for bf16, 8-byte for fp32).
__device__ __forceinline__ void load2(const __bf16* p, float& a, float& b) {
  const uint32_t u = *reinterpret_cast<const uint32_t*>(p);
  a = __uint_as_float(u << 16);
  b = __uint_as_float(u & 0xffff0000u);
}
__device__ __forceinline__ void load2(const float* p, float& a, float& b) {
  const float2 f = *reinterpret_cast<const float2*>(p);
  a = f.x;
  b = f.y;
}

// Per (chunk, QK head): the normalised key and query rows, zero past the end.
// Lane l holds elements D/64 l .. of a row (one 4- or 8-byte access each way).
template <typename T>
__global__ __launch_bounds__(256) void bwd_stage_qk_kernel(BwdWs w, const T* q, const T* k, int64_t qs,
                                                           int64_t ks, int h_qk, int D, int C, int l2norm) {
  const int gc = blockIdx.x / h_qk, hq = blockIdx.x % h_qk;
  if (gc >= *w.nc) return;
  const ChunkRec cr = w.ct[gc];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, per = D / 64, c0 = per * lane;
  float* Kn = w.Kn + ((int64_t)gc * h_qk + hq) * C * D;
  float* Qn = w.Qn + ((int64_t)gc * h_qk + hq) * C * D;
  // a wave takes 4 rows at a time, all their loads issued before the sums
  for (int r0 = 4 * wave; r0 < C; r0 += 16) {
    float v[4][2][2];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
#pragma unroll
      for (int which = 0; which < 2; ++which) {
        const int r = r0 + rr;
        v[rr][which][0] = v[rr][which][1] = 0.f;
        if (r < cr.len) {
          const T* src = (which ? q : k) + (int64_t)(cr.t0 + r) * (which ? qs : ks) + (int64_t)hq * D + c0;
          if (per == 2) load2(src, v[rr][which][0], v[rr][which][1]);
          else v[rr][which][0] = to_f32(src[0]);
        }
      }
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
#pragma unroll
      for (int which = 0; which < 2; ++which) {
        const int r = r0 + rr;
        const float ss = wave_sum(v[rr][which][0] * v[rr][which][0] + v[rr][which][1] * v[rr][which][1]);
        const float rn = (l2norm && r < cr.len) ? 1.0f / sqrtf(ss + 1e-6f) : 1.0f;
        float* dst = (which ? Qn : Kn) + (int64_t)r * D + c0;
        if (per == 2) *reinterpret_cast<float2*>(dst) = make_float2(v[rr][which][0] * rn, v[rr][which][1] * rn);
        else dst[0] = v[rr][which][0] * rn;
      }
  }
}

// ----------------------------------------- prep: gates, T, Pm, scaled rows
// Per (chunk, V head): G, gam, e, beta; T = (I + A)^-1 by forward
// substitution; Pm; the row scalings of K^ and Q^ (vec rows); beta V and dO.
template <typename T>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdWs w, const float* g, const float* beta, const T* v,
                                                       int64_t vs, const T* d_o, int h_qk, int h_v, int D,
                                                       int C, float scale, int erase) {
  const int gc = blockIdx.x / h_v, h = blockIdx.x % h_v;
  if (gc >= *w.nc) return;
  const ChunkRec cr = w.ct[gc];
  const int hq = h / (h_v / h_qk), tid = threadIdx.x;
  const int64_t bv = (int64_t)gc * h_v + h, bq = (int64_t)gc * h_qk + hq;
  __shared__ float sG[64], sGam[64], sE[64], sB[64];
  __shared__ float sA[64][65];
  __shared__ float sT[64][65];
  if (tid < 64) {  // G = cumsum(g): an inclusive scan over the lanes of wave 0
    const int r = tid;
    const bool in = r < cr.len;
    float x = in ? g[(int64_t)(cr.t0 + r) * h_v + h] : 0.f;
#pragma unroll
    for (int off = 1; off < 64; off *= 2) {
      const float t = __shfl_up(x, off, 64);
      if (r >= off) x += t;
    }
    if (r < C) {
      sG[r] = x;
      sB[r] = in ? beta[(int64_t)(cr.t0 + r) * h_v + h] : 0.f;
    }
  }
  __syncthreads();
  float* vec = w.vec + bv * kNVec * C;
  for (int r = tid; r < C; r += blockDim.x) {
    sGam[r] = expf(sG[r]);
    sE[r] = expf(sG[C - 1] - sG[r]);
    vec[kVecG * C + r] = sG[r];
    vec[kVecGam * C + r] = sGam[r];
    vec[kVecE * C + r] = sE[r];
    vec[kVecBeta * C + r] = sB[r];
    vec[kVecBG * C + r] = erase ? sB[r] * sGam[r] : 0.f;
    vec[kVecSG * C + r] = scale * sGam[r];
  }
  const float* KK = w.KK + bq * C * C;
  const float* QK = w.QK + bq * C * C;
  float* Pm = w.cc[cPm] + bv * C * C;
  for (int e = tid; e < C * C; e += blockDim.x) {
    const int r = e / C, j = e % C;
    sA[r][j] = (erase && j < r) ? sB[r] * expf(sG[r] - sG[j]) * KK[e] : 0.f;
    Pm[e] = j <= r ? scale * expf(sG[r] - sG[j]) * QK[e] : 0.f;
  }
  __syncthreads();
  // (I + A) T = I, A strictly lower: row i of T is e_i - sum_{j<i} A_ij T_j.
  // Lane c of wave 0 solves column c alone (it reads back only its own
  // writes, and A is read-only here), so the rows need no barrier; the other
  // waves meanwhile write beta V and dO in the chunk layout (the row scalings
  // of K^ and Q^ are applied where they are read).
  if (tid < 64) {
    if (tid < C)
      for (int i = 0; i < C; ++i) {
        float s = i == tid ? 1.f : 0.f;
        for (int j = 0; j < i; ++j) s -= sA[i][j] * sT[j][tid];
        sT[i][tid] = s;
      }
  } else {
    float* BV = w.cd[mBV] + bv * C * D;
    float* DO = w.cd[mDO] + bv * C * D;
    for (int e = 4 * (tid - 64); e < C * D; e += 4 * (blockDim.x - 64)) {
      const int r = e / D, c = e % D;
      const bool in = r < cr.len;
      const int64_t tok = (int64_t)(cr.t0 + r);
      float vv[4] = {0.f, 0.f, 0.f, 0.f}, dd[4] = {0.f, 0.f, 0.f, 0.f};
      if (in) {
        load4(v + tok * vs + (int64_t)h * D + c, vv);
        load4(d_o + (tok * h_v + h) * D + c, dd);
      }
      *reinterpret_cast<v4f*>(BV + e) = v4f{sB[r] * vv[0], sB[r] * vv[1], sB[r] * vv[2], sB[r] * vv[3]};
      *reinterpret_cast<v4f*>(DO + e) = v4f{dd[0], dd[1], dd[2], dd[3]};
    }
  }
  __syncthreads();
  float* Tm = w.cc[cT] + bv * C * C;
  for (int e = tid; e < C * C; e += blockDim.x) Tm[e] = sT[e / C][e % C];
}

// ----------------------------------------------------------------- chain
// One workgroup per (sequence, V head, 16 state columns) and direction.  Per
// chunk, with Y the D x 16 state slice:
//   forward: store Y as X_c;   U  = Ut  - W Y;         Y = gam Y + EK^T U
//   reverse: store Y as dX'_c; dU = PdO + EK Y;        Y = gam Y + Z - W^T dU
// (chunks in reverse order).  Y starts from the initial state (forward) or
// the final-state gradient (reverse); the reverse chain's last Y is the
// initial-state gradient.  The two directions need nothing from each other
// (the reverse chain reads only the recomputed chunk quantities), so one
// launch runs both.  The next chunk's two C x D operands are fetched into
// registers while the current chunk computes.
constexpr int kCW = 16;
// W and diag(e) K^ of one chunk (e K^ formed from the QK head's rows of K^)
template <bool REV, int NPF>
__device__ __forceinline__ void chain_fetch(const BwdWs& w, int gc, int h, int h_v, int h_qk, int D, int C,
                                            int tid, v4f (&r1)[NPF], v4f (&r2)[NPF]) {
  const int64_t b = (int64_t)gc * h_v + h, bq = (int64_t)gc * h_qk + h / (h_v / h_qk);
  const v4f* pw = reinterpret_cast<const v4f*>(w.cd[mW] + b * C * D);
  const v4f* pk = reinterpret_cast<const v4f*>(w.Kn + bq * C * D);
  const float* e = w.vec + b * kNVec * C + kVecE * C;
#pragma unroll
  for (int u = 0; u < NPF; ++u) {
    const int q = tid + 256 * u;
    const v4f wv = pw[q], ek = e[q / (D / 4)] * pk[q];
    r1[u] = REV ? ek : wv;
    r2[u] = REV ? wv : ek;
  }
}

template <bool REV, int D, int C>
__device__ __forceinline__ void chain_body(const BwdWs& w, const float* s_in, float* s_out, int h_v, int h_qk) {
  const int n = blockIdx.x / h_v, h = blockIdx.x % h_v, col0 = blockIdx.y * kCW, tid = threadIdx.x;
  extern __shared__ float lds[];
  constexpr int LP = D + 4;    // P1 row pitch: the 16 rows a wave reads fall in distinct banks
  float* P1 = lds;             // C x LP
  float* P2 = P1 + C * LP;     // C x D
  float* Y = P2 + C * D;       // D x 16
  float* Uv = Y + D * kCW;     // C x 16
  for (int e = tid; e < D * kCW; e += 256) {
    const int k = e / kCW, c = e % kCW;
    Y[e] = s_in ? s_in[(((int64_t)n * h_v + h) * D + col0 + c) * D + k] : 0.f;
  }
  const int c_lo = w.co[n], c_hi = w.co[n + 1];
  constexpr int NPF = C * D / 1024;  // float4 per thread per operand
  constexpr int NPT = D / 16;             // state outputs per thread
  constexpr int TPR = kCW / NPT;          // threads per state row
  const int yk = tid / TPR, yc = (tid % TPR) * NPT;
  v4f r1[NPF], r2[NPF];
  const int nchunks = c_hi - c_lo;
  if (nchunks > 0) chain_fetch<REV, NPF>(w, REV ? c_hi - 1 : c_lo, h, h_v, h_qk, D, C, tid, r1, r2);
  for (int i = 0; i < nchunks; ++i) {
    const int gc = REV ? c_hi - 1 - i : c_lo + i;
    const int64_t b = (int64_t)gc * h_v + h;
    lds_barrier();  // the previous chunk is done with P1, P2, Uv and Y
#pragma unroll
    for (int u = 0; u < NPF; ++u) {
      const int q = tid + 256 * u;
      *reinterpret_cast<v4f*>(P1 + (q / (D / 4)) * LP + (q % (D / 4)) * 4) = r1[u];
      reinterpret_cast<v4f*>(P2)[q] = r2[u];
    }
    if (i + 1 < nchunks) chain_fetch<REV, NPF>(w, REV ? gc - 1 : gc + 1, h, h_v, h_qk, D, C, tid, r1, r2);
    float* ys = w.dd[REV ? xDXs : xXs] + b * D * D;
    for (int e = tid; e < D * kCW; e += 256) ys[(int64_t)(e / kCW) * D + col0 + e % kCW] = Y[e];
    lds_barrier();
    // R1 = P1 Y, then U = Vb -/+ R1 (C x 16)
    const float* vb = w.cd[REV ? mPdO : mUt] + b * C * D;
    float* uo = w.cd[REV ? mDU : mU] + b * C * D;
    for (int e = tid; e < C * (kCW / 4); e += 256) {
      const int r = e / (kCW / 4), c4 = (e % (kCW / 4)) * 4;
      float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
      for (int k0 = 0; k0 < D; k0 += 8) {
        float pk[8];
        v4f y[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          pk[u] = P1[r * LP + k0 + u];
          y[u] = *reinterpret_cast<const v4f*>(&Y[(k0 + u) * kCW + c4]);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          a0 = fmaf(pk[u], y[u].x, a0);
          a1 = fmaf(pk[u], y[u].y, a1);
          a2 = fmaf(pk[u], y[u].z, a2);
          a3 = fmaf(pk[u], y[u].w, a3);
        }
      }
      const float4 v = *reinterpret_cast<const float4*>(vb + (int64_t)r * D + col0 + c4);
      const float4 u = REV ? make_float4(v.x + a0, v.y + a1, v.z + a2, v.w + a3)
                           : make_float4(v.x - a0, v.y - a1, v.z - a2, v.w - a3);
      *reinterpret_cast<float4*>(&Uv[r * kCW + c4]) = u;
      *reinterpret_cast<float4*>(uo + (int64_t)r * D + col0 + c4) = u;
    }
    lds_barrier();
    // Y = gam Y +/- P2^T U (+ Z)
    const float gam = w.vec[b * kNVec * C + kVecGam * C + C - 1];
    float acc[NPT];
#pragma unroll
    for (int j = 0; j < NPT; ++j) acc[j] = 0.f;
    for (int r0 = 0; r0 < C; r0 += 4) {
      float pk[4];
      v4f uv[4][NPT / 4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        pk[u] = P2[(r0 + u) * D + yk];
#pragma unroll
        for (int q = 0; q < NPT / 4; ++q) uv[u][q] = *reinterpret_cast<const v4f*>(&Uv[(r0 + u) * kCW + yc + 4 * q]);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int q = 0; q < NPT / 4; ++q) {
          acc[4 * q + 0] = fmaf(pk[u], uv[u][q].x, acc[4 * q + 0]);
          acc[4 * q + 1] = fmaf(pk[u], uv[u][q].y, acc[4 * q + 1]);
          acc[4 * q + 2] = fmaf(pk[u], uv[u][q].z, acc[4 * q + 2]);
          acc[4 * q + 3] = fmaf(pk[u], uv[u][q].w, acc[4 * q + 3]);
        }
    }
    if constexpr (REV) {
      const float* z = w.dd[xZ] + b * D * D + (int64_t)yk * D + col0 + yc;
#pragma unroll
      for (int j = 0; j < NPT; ++j) Y[yk * kCW + yc + j] = gam * Y[yk * kCW + yc + j] + z[j] - acc[j];
    } else {
#pragma unroll
      for (int j = 0; j < NPT; ++j) Y[yk * kCW + yc + j] = gam * Y[yk * kCW + yc + j] + acc[j];
    }
  }
  if (REV && s_out) {
    lds_barrier();
    for (int e = tid; e < D * kCW; e += 256) {
      const int k = e / kCW, c = e % kCW;
      s_out[(((int64_t)n * h_v + h) * D + col0 + c) * D + k] = Y[e];
    }
  }
}

template <int D, int C>
__global__ __launch_bounds__(256) void bwd_chains_kernel(BwdWs w, const float* s0, const float* dsf, float* ds0,
                                                         int h_v, int h_qk) {
  if (blockIdx.z == 0) chain_body<false, D, C>(w, s0, nullptr, h_v, h_qk);
  else chain_body<true, D, C>(w, dsf, ds0, h_v, h_qk);
}

template <int D, int C>
hipError_t launch_chains(const BwdWs& w, const PrefillBwdParams& p, hipStream_t stream) {
  const size_t lds = (C * (D + 4) + C * D + D * kCW + C * kCW) * sizeof(float);
  const void* f = reinterpret_cast<const void*>(bwd_chains_kernel<D, C>);
  hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_chains_kernel<D, C>), dim3((unsigned)(p.n_seqs * p.h_v), D / kCW, 2), dim3(256), lds,
                     stream, w, p.initial_state, p.d_final_state, p.d_initial_state, p.h_v, p.h_qk);
  return hipGetLastError();
}

// ---------------------------------------------------- chain, bf16 operands
// The same two chains for bf16 inputs, on bf16 MFMA (16x16x32): the chunk
// operands and the state slice are rounded to bf16 as MFMA operands (as the
// forward scan does with its state), while the state itself, U and every
// stored result stay fp32.  One wave per 16 state columns; the four waves of
// a workgroup share one bf16 LDS copy of the chunk's two C x D operands, both
// row-major.  A 32-deep k-step takes k = 4g + j (j < 4), then 16 + 4g + j - 4
// (g = lane / 16): the accumulator tiles 2s and 2s + 1 of Y (or of U) are the
// B operand as they stand, R = P1 Y reads rows of P1, and the update reads
// P1-shaped tiles of P2 transposed (ds_read_b64_tr_b16).
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4v lds_short4v;

__device__ __forceinline__ bf16x8_t frag_rows(const __bf16* row, int g, bool half) {
  const uint2 lo = *reinterpret_cast<const uint2*>(row + 4 * g);
  const uint2 hi = half ? make_uint2(0u, 0u) : *reinterpret_cast<const uint2*>(row + 16 + 4 * g);
  return __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
}
// m = column c0 + l16 of a row-major tile, k = rows r0 + 4g + {0..3} (+16)
__device__ __forceinline__ bf16x8_t frag_cols(const __bf16* P, int ld, int r0, int c0, int l16, int g, bool half) {
  const __bf16* p = P + (r0 + 4 * g + (l16 >> 2)) * ld + c0 + 4 * (l16 & 3);
  const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)(__attribute__((address_space(3))) __bf16*)(p));
  short4v hi = {0, 0, 0, 0};
  if (!half)
    hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_short4v*)(__attribute__((address_space(3))) __bf16*)(p + 16 * ld));
  const uint2 a = __builtin_bit_cast(uint2, lo), b = __builtin_bit_cast(uint2, hi);
  return __builtin_bit_cast(bf16x8_t, make_uint4(a.x, a.y, b.x, b.y));
}
__device__ __forceinline__ bf16x8_t frag_acc(const v4f& a, const v4f& b) {
  return __builtin_bit_cast(bf16x8_t, make_uint4(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]),
                                                 pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3])));
}

constexpr int kBCols = 64;  // state columns per workgroup (16 per wave)

template <bool REV, int D, int C>
__device__ __forceinline__ void chain_rows16(const BwdWs& w, int gc, int h, int h_v, int col, int g4,
                                             float (&vb)[C / 16][4], float (&zz)[D / 16][4]) {
  const int64_t b = (int64_t)gc * h_v + h;
  const float* v = w.cd[REV ? mPdO : mUt] + b * C * D + col;
#pragma unroll
  for (int rb = 0; rb < C / 16; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) vb[rb][i] = v[(int64_t)(16 * rb + 4 * g4 + i) * D];
  if constexpr (REV) {
    const float* z = w.dd[xZ] + b * D * D + col;
#pragma unroll
    for (int kb = 0; kb < D / 16; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) zz[kb][i] = z[(int64_t)(16 * kb + 4 * g4 + i) * D];
  }
}

template <bool REV, int D, int C>
__device__ __forceinline__ void chain_body_bf16(const BwdWs& w, const float* s_in, float* s_out, int h_v,
                                                int h_qk) {
  constexpr int NR = C / 16, NK = D / 16, NPF = C * D / 1024, LD = D + 8;
  constexpr int NRS = (C + 31) / 32;   // 32-deep k-steps over the chunk rows
  constexpr bool HALF = C == 16;
  const int n = blockIdx.x / h_v, h = blockIdx.x % h_v, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, l16 = lane & 15, g4 = lane >> 4;
  const int col = blockIdx.y * kBCols + 16 * wave + l16;
  extern __shared__ float lds[];
  __bf16* P1 = reinterpret_cast<__bf16*>(lds);  // C x LD
  __bf16* P2 = P1 + C * LD;                      // C x LD
  const int64_t srow = (((int64_t)n * h_v + h) * D + col) * D;
  v4f Y[NK];
#pragma unroll
  for (int kb = 0; kb < NK; ++kb)
#pragma unroll
    for (int i = 0; i < 4; ++i) Y[kb][i] = s_in ? s_in[srow + 16 * kb + 4 * g4 + i] : 0.f;
  const int c_lo = w.co[n], c_hi = w.co[n + 1], nchunks = c_hi - c_lo;
  v4f r1[NPF], r2[NPF];
  float vb[NR][4], zz[NK][4];
  if (nchunks > 0) {
    chain_fetch<REV, NPF>(w, REV ? c_hi - 1 : c_lo, h, h_v, h_qk, D, C, tid, r1, r2);
    chain_rows16<REV, D, C>(w, REV ? c_hi - 1 : c_lo, h, h_v, col, g4, vb, zz);
  }
  const v4f zero4 = {0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < nchunks; ++i) {
    const int gc = REV ? c_hi - 1 - i : c_lo + i;
    const int64_t b = (int64_t)gc * h_v + h;
    lds_barrier();  // every wave is done with the previous chunk's P1, P2
#pragma unroll
    for (int u = 0; u < NPF; ++u) {
      const int q = tid + 256 * u, r = q / (D / 4), k4 = (q % (D / 4)) * 4;
      *reinterpret_cast<uint2*>(P1 + r * LD + k4) =
          make_uint2(pack_bf16x2(r1[u][0], r1[u][1]), pack_bf16x2(r1[u][2], r1[u][3]));
      *reinterpret_cast<uint2*>(P2 + r * LD + k4) =
          make_uint2(pack_bf16x2(r2[u][0], r2[u][1]), pack_bf16x2(r2[u][2], r2[u][3]));
    }
    if (i + 1 < nchunks) chain_fetch<REV, NPF>(w, REV ? gc - 1 : gc + 1, h, h_v, h_qk, D, C, tid, r1, r2);
    float* ys = w.dd[REV ? xDXs : xXs] + b * D * D + col;
#pragma unroll
    for (int kb = 0; kb < NK; ++kb)
#pragma unroll
      for (int j = 0; j < 4; ++j) ys[(int64_t)(16 * kb + 4 * g4 + j) * D] = Y[kb][j];
    lds_barrier();
    // R = P1 Y (C x 16), then U = Vb -/+ R
    v4f R[NR];
#pragma unroll
    for (int rb = 0; rb < NR; ++rb) R[rb] = zero4;
#pragma unroll
    for (int kp = 0; kp < NK / 2; ++kp) {
      const bf16x8_t bop = frag_acc(Y[2 * kp], Y[2 * kp + 1]);
#pragma unroll
      for (int rb = 0; rb < NR; ++rb)
        R[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(frag_rows(P1 + (16 * rb + l16) * LD + 32 * kp, g4, false),
                                                        bop, R[rb], 0, 0, 0);
    }
    float* uo = w.cd[REV ? mDU : mU] + b * C * D + col;
#pragma unroll
    for (int rb = 0; rb < NR; ++rb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        R[rb][j] = REV ? vb[rb][j] + R[rb][j] : vb[rb][j] - R[rb][j];
        uo[(int64_t)(16 * rb + 4 * g4 + j) * D] = R[rb][j];
      }
    // Y = gam Y (+ Z) +/- P2^T U
    const float gam = w.vec[b * kNVec * C + kVecGam * C + C - 1];
#pragma unroll
    for (int kb = 0; kb < NK; ++kb)
#pragma unroll
      for (int j = 0; j < 4; ++j) Y[kb][j] = gam * Y[kb][j] + (REV ? zz[kb][j] : 0.f);
#pragma unroll
    for (int rp = 0; rp < NRS; ++rp) {
      v4f ua = R[2 * rp], ub = HALF ? zero4 : R[(2 * rp + 1) < NR ? 2 * rp + 1 : 0];
      if (REV) {
        ua = -ua;
        ub = -ub;
      }
      const bf16x8_t bop = frag_acc(ua, ub);
#pragma unroll
      for (int kb = 0; kb < NK; ++kb)
        Y[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(frag_cols(P2, LD, 32 * rp, 16 * kb, l16, g4, HALF), bop,
                                                        Y[kb], 0, 0, 0);
    }
    if (i + 1 < nchunks) chain_rows16<REV, D, C>(w, REV ? gc - 1 : gc + 1, h, h_v, col, g4, vb, zz);
  }
  if (REV && s_out) {
#pragma unroll
    for (int kb = 0; kb < NK; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) s_out[srow + 16 * kb + 4 * g4 + i] = Y[kb][i];
  }
}

template <int D, int C>
__global__ __launch_bounds__(256) void bwd_chains_bf16_kernel(BwdWs w, const float* s0, const float* dsf,
                                                              float* ds0, int h_v, int h_qk) {
  if (blockIdx.z == 0) chain_body_bf16<false, D, C>(w, s0, nullptr, h_v, h_qk);
  else chain_body_bf16<true, D, C>(w, dsf, ds0, h_v, h_qk);
}

template <int D, int C>
hipError_t launch_chains_bf16(const BwdWs& w, const PrefillBwdParams& p, hipStream_t stream) {
  const size_t lds = (size_t)2 * C * (D + 8) * sizeof(__bf16);
  hipLaunchKernelGGL((bwd_chains_bf16_kernel<D, C>), dim3((unsigned)(p.n_seqs * p.h_v), D / kBCols, 2), dim3(256),
                     lds, stream, w, p.initial_state, p.d_final_state, p.d_initial_state, p.h_v, p.h_qk);
  return hipGetLastError();
}

// ------------------------------------------------ chunk-local, one kernel
// Per (chunk, V head), once the chains have stored X_c, dX'_c, U and dU:
// every chunk-local gradient in one workgroup on fp32 MFMA (16x16x4), so the
// C x d and C x C intermediates never leave the CU.  4 NP waves: wave w
// owns rows 16 (w % 4) .. +15 of every C-row result and one of NP column
// parts (w / 4), so a tile row sum is NP partials and the dK^
// and dQ^ tiles accumulate in registers across the products.  dU, U, dO and
// T sit in LDS (U's and dO's space is reused for dW and dT T^T once they are
// done); X and dX' are read as MFMA operands straight from memory.
//   dPm = dO U^T -> dQK = scale Gam o dPm (lower incl.)
//   T^T dU -> dv = diag(beta) T^T dU, and dbeta's V term
//   dT = dU (diag(beta) V)^T + dW (diag(beta gam) K^)^T,  dW = -dU X^T
//   dO X^T -> dQ^ += scale diag(gam) dO X^T, and dG's gam term
//   U dX'^T -> dK^ += diag(e) U dX'^T
//   dA = -T^T dT T^T -> dKK = beta Gam o dA (strict lower)
//   T^T dW -> dK^ += diag(beta gam) T^T dW, and the beta gam terms
//   dK^ += dQK^T Q^ + (dKK + dKK^T) K^,  dQ^ += dQK K^
// then dG (with the Gam row and column sums), its reverse cumulative sum dg,
// and dbeta.  MFMA lane l supplies A[l % 16][l / 16] and B[l / 16][l % 16]
// of a 16 x 4 / 4 x 16 slice and holds C rows 4 (l / 16) .. +3 of column
// l % 16; row16_sum adds a tile row over its 16 columns.
// Per-row scalars: G, gam, e, beta, beta gam, scale gam, u, then one partial
// per column part (NP of them) each of Q^ . dO X^T, K^ . T^T dW, V . T^T dU,
// the dbeta part of dA and the Gam terms' row sums.
enum { lG = 0, lGam, lE, lBeta, lBG, lSG, lU };

template <int D, int C, int NP>
struct LocalLayout {
  static constexpr int lA = lU + 1, lS = lA + NP, lB = lS + NP, lDB = lB + NP, lR = lDB + NP, nRows = lR + NP;
  static constexpr int P1 = D + 4, P2 = C + 4;
  static constexpr int oDU = 0, oU = oDU + C * P1, oDO = oU + C * P1, oT = oDO + C * P1, oX = oT + C * P2,
                       oY = oX + C * P2, oV = oY + C * P2, oCol = oV + nRows * C, oRed = oCol + 4 * C,
                       floats = oRed + 4 * NP;
};

__device__ __forceinline__ v4f mma4(float a, float b, const v4f& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// acc[nt] += sum_k A[r][k] B[16 nt + n][k] for this lane's tile row r, with
// both operands stored k-contiguous (a: this lane's row of A; b: the first
// B row of the tiles).  Lane (l16, g4) takes k = k0 + 4 g4 + j into MFMA j,
// the same permutation of k for both operands, so each operand arrives in
// one 16-byte load.
template <int NT>
__device__ __forceinline__ void mm_kk(v4f (&acc)[NT], const float* a, const float* b, int ldb, int K, int l16,
                                      int g4) {
  for (int k0 = 0; k0 < K; k0 += 16) {
    const v4f av = *reinterpret_cast<const v4f*>(a + k0 + 4 * g4);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const v4f bv = *reinterpret_cast<const v4f*>(b + (int64_t)(16 * nt + l16) * ldb + k0 + 4 * g4);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[nt] = mma4(av[j], bv[j], acc[nt]);
    }
  }
}

// acc[nt] += sum_k At[k][r] B[k][16 nt + n] (A stored transposed: at points
// at column r of At; B stored k-major from its first tile column).
template <int NT>
__device__ __forceinline__ void mm_tn(v4f (&acc)[NT], const float* at, int lda, const float* b, int ldb, int K,
                                      int l16, int g4) {
#pragma unroll 4
  for (int k0 = 0; k0 < K; k0 += 4) {
    const float av = at[(k0 + g4) * lda];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] = mma4(av, b[(k0 + g4) * ldb + 16 * nt + l16], acc[nt]);
  }
}

// Sum over the 4 lane groups of a wave (the 16 rows of a tile column held in
// lanes l16, l16 + 16, l16 + 32, l16 + 48).
__device__ __forceinline__ float col4_sum(float x) {
  x += __shfl_xor(x, 16, 64);
  x += __shfl_xor(x, 32, 64);
  return x;
}

template <typename T, int D, int C, int NP>
__global__ __launch_bounds__(256 * NP) void bwd_local_kernel(BwdWs w, const T* v, int64_t vs, T* dv, int64_t dvs,
                                                        float* dg, float* dbeta, int h_qk, int h_v, float scale,
                                                        int erase, const T* qx, const T* kx, int64_t qs, int64_t ks,
                                                        T* dq, T* dk, int64_t dqs, int64_t dks, int l2norm,
                                                        int direct) {
  using L = LocalLayout<D, C, NP>;
  // NH tiles of d columns per wave; the C x C products split into NCP parts
  // of NCH tiles (NCP < NP when C has fewer tiles than there are parts)
  constexpr int P1 = L::P1, P2 = L::P2, NN = D / 16, NC = C / 16, NH = NN / NP;
  constexpr int NCP = NC < NP ? NC : NP, NCH = NC / NCP, NT = 256 * NP, RPW = 16 / NP;
  const int gc = blockIdx.x / h_v, h = blockIdx.x % h_v, tid = threadIdx.x;
  if (gc >= *w.nc) return;
  const ChunkRec cr = w.ct[gc];
  const int hq = h / (h_v / h_qk), lane = tid & 63, wave = tid >> 6, l16 = lane & 15, g4 = lane >> 4;
  const int mt = wave & 3, ch = wave >> 2, r0 = 16 * mt, cb = ch * (D / NP), jb = 16 * NCH * ch;
  const bool rows = mt < NC, ccw = rows && ch < NCP;
  const int64_t bv = (int64_t)gc * h_v + h, bq = (int64_t)gc * h_qk + hq;
  extern __shared__ float lds[];
  float* sDU = lds + L::oDU;
  float* sU = lds + L::oU;    // U, then dW
  float* sDO = lds + L::oDO;  // dO, then dT T^T
  float* sT = lds + L::oT;
  float* sX = lds + L::oX;    // dQK
  float* sY = lds + L::oY;    // dT, then dKK
  float* sV = lds + L::oV;    // per-row scalars, nRows x C
  float* sCol = lds + L::oCol;  // column sums of the Gam terms per row tile, 4 x C
  float* sRed = lds + L::oRed;
  const float* gDU = w.cd[mDU] + bv * C * D;
  const float* gU = w.cd[mU] + bv * C * D;
  const float* gDO = w.cd[mDO] + bv * C * D;
  const float* gBV = w.cd[mBV] + bv * C * D;
  const float* gPdO = w.cd[mPdO] + bv * C * D;
  const float* gT = w.cc[cT] + bv * C * C;
  const float* gKK = w.KK + bq * C * C;
  const float* gQK = w.QK + bq * C * C;
  const float* gKn = w.Kn + bq * C * D;
  const float* gQn = w.Qn + bq * C * D;
  const float* gXs = w.dd[xXs] + bv * D * D;
  const float* gdXs = w.dd[xDXs] + bv * D * D;
  const float* vec = w.vec + bv * kNVec * C;
  // ---- stage dU, U, dO, T and the per-row scalars
  for (int e = 4 * tid; e < C * D; e += 4 * NT) {
    const int r = e / D, c = e % D;
    *reinterpret_cast<v4f*>(sDU + r * P1 + c) = *reinterpret_cast<const v4f*>(gDU + e);
    *reinterpret_cast<v4f*>(sU + r * P1 + c) = *reinterpret_cast<const v4f*>(gU + e);
    *reinterpret_cast<v4f*>(sDO + r * P1 + c) = *reinterpret_cast<const v4f*>(gDO + e);
  }
  for (int e = 4 * tid; e < C * C; e += 4 * NT)
    *reinterpret_cast<v4f*>(sT + (e / C) * P2 + e % C) = *reinterpret_cast<const v4f*>(gT + e);
  for (int e = tid; e < C; e += NT) {
    sV[lG * C + e] = vec[kVecG * C + e];
    sV[lGam * C + e] = vec[kVecGam * C + e];
    sV[lE * C + e] = vec[kVecE * C + e];
    sV[lBeta * C + e] = vec[kVecBeta * C + e];
    sV[lBG * C + e] = vec[kVecBG * C + e];
    sV[lSG * C + e] = vec[kVecSG * C + e];
#pragma unroll
    for (int q = lU; q < L::nRows; ++q) sV[q * C + e] = 0.f;
  }
  lds_barrier();
  const v4f z4 = {0.f, 0.f, 0.f, 0.f};
  v4f accK[NH], accQ[NH], accW[NH];
  float xk[NH][4], xq[NH][4];
  if (ccw) {
    // ---- dPm = dO U^T -> dQK = scale Gam o dPm (lower incl.); Gam terms of dG
    v4f acc[NCH];
#pragma unroll
    for (int nt = 0; nt < NCH; ++nt) acc[nt] = z4;
    mm_kk<NCH>(acc, sDO + (r0 + l16) * P1, sU + jb * P1, P1, D, l16, g4);
    float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nt = 0; nt < NCH; ++nt) {
      const int j = jb + 16 * nt + l16;
      float cs = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = r0 + 4 * g4 + i;
        const float dq = j <= r ? scale * expf(sV[lG * C + r] - sV[lG * C + j]) * acc[nt][i] : 0.f;
        sX[r * P2 + j] = dq;
        const float gg = gQK[r * C + j] * dq;
        rs[i] += gg;
        cs += gg;
      }
      cs = col4_sum(cs);
      if (g4 == 0) sCol[mt * C + j] = cs;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x = row16_sum(rs[i]);
      if (l16 == 0) sV[(L::lR + ch) * C + r0 + 4 * g4 + i] = x;
    }
  }
  if (rows) {
    // ---- T^T dU -> dv = diag(beta) T^T dU, and dbeta's V term
    {
#pragma unroll
      for (int nt = 0; nt < NH; ++nt) accW[nt] = z4;
      mm_tn<NH>(accW, sT + r0 + l16, P2, sDU + cb, P1, C, l16, g4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = r0 + 4 * g4 + i;
        const bool in = r < cr.len;
        const float be = sV[lBeta * C + r];
        const int64_t tok = (int64_t)(cr.t0 + r);
        float b1 = 0.f;
#pragma unroll
        for (int nt = 0; nt < NH; ++nt) {
          const int c = cb + 16 * nt + l16;
          if (in) {
            b1 += to_f32(v[tok * vs + (int64_t)h * D + c]) * accW[nt][i];
            dv[tok * dvs + (int64_t)h * D + c] = from_f32<T>(be * accW[nt][i]);
          }
        }
        b1 = row16_sum(b1);
        if (l16 == 0) sV[(L::lB + ch) * C + r] = b1;
      }
    }
    // ---- dT = dU (diag(beta) V)^T; the dW term is added below
    if (ccw) {
      v4f acc[NCH];
#pragma unroll
      for (int nt = 0; nt < NCH; ++nt) acc[nt] = z4;
      mm_kk<NCH>(acc, sDU + (r0 + l16) * P1, gBV + (int64_t)jb * D, D, D, l16, g4);
#pragma unroll
      for (int nt = 0; nt < NCH; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) sY[(r0 + 4 * g4 + i) * P2 + jb + 16 * nt + l16] = acc[nt][i];
    }
    // ---- dO X^T and dW = -dU X^T (X stored [d_k][d_v], so B[n][k] = X[n][k] is k-contiguous)
    {
#pragma unroll
      for (int nt = 0; nt < NH; ++nt) {
        accQ[nt] = z4;
        accW[nt] = z4;
      }
      const float* ao = sDO + (r0 + l16) * P1;
      const float* aw = sDU + (r0 + l16) * P1;
      const float* bx = gXs + (int64_t)(cb + l16) * D;
      for (int k0 = 0; k0 < D; k0 += 16) {
        const v4f a1 = *reinterpret_cast<const v4f*>(ao + k0 + 4 * g4);
        const v4f a2 = *reinterpret_cast<const v4f*>(aw + k0 + 4 * g4);
#pragma unroll
        for (int nt = 0; nt < NH; ++nt) {
          const v4f b = *reinterpret_cast<const v4f*>(bx + (int64_t)16 * nt * D + k0 + 4 * g4);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            accQ[nt] = mma4(a1[j], b[j], accQ[nt]);
            accW[nt] = mma4(a2[j], b[j], accW[nt]);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = r0 + 4 * g4 + i;
        const float sg = sV[lSG * C + r];
        float a = 0.f;
#pragma unroll
        for (int nt = 0; nt < NH; ++nt) {
          a += gQn[r * D + cb + 16 * nt + l16] * accQ[nt][i];
          accQ[nt][i] *= sg;  // dQ^ starts as scale gam dO X^T
          accW[nt][i] = -accW[nt][i];
        }
        a = row16_sum(a);
        if (l16 == 0) sV[(L::lA + ch) * C + r] = a;
      }
    }
    // ---- dK^ starts as diag(e) U dX'^T; u_r = U_r . (dU_r - (Pm^T dO)_r)
    {
#pragma unroll
      for (int nt = 0; nt < NH; ++nt) accK[nt] = z4;
      mm_kk<NH>(accK, sU + (r0 + l16) * P1, gdXs + (int64_t)cb * D, D, D, l16, g4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ee = sV[lE * C + r0 + 4 * g4 + i];
#pragma unroll
        for (int nt = 0; nt < NH; ++nt) accK[nt][i] *= ee;
      }
      for (int rr = 0; rr < RPW; ++rr) {
        const int r = r0 + RPW * ch + rr;
        float u = 0.f;
        for (int c = lane; c < D; c += 64) u += sU[r * P1 + c] * (sDU[r * P1 + c] - gPdO[r * D + c]);
        u = wave_sum(u);
        if (lane == 0) sV[lU * C + r] = u;
      }
    }
  }
  // <X, dX'> over the whole d_k x d_v block (every wave)
  {
    float xd = 0.f;
    for (int e = 4 * tid; e < D * D; e += 4 * NT) {
      const v4f x4 = *reinterpret_cast<const v4f*>(gXs + e), d4 = *reinterpret_cast<const v4f*>(gdXs + e);
      xd += x4[0] * d4[0] + x4[1] * d4[1] + x4[2] * d4[2] + x4[3] * d4[3];
    }
    xd = wave_sum(xd);
    if (lane == 0) sRed[wave] = xd;
  }
  lds_barrier();  // every wave is done with U and dO
  float* sW = sU;
  if (rows) {
#pragma unroll
    for (int nt = 0; nt < NH; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) sW[(r0 + 4 * g4 + i) * P1 + cb + 16 * nt + l16] = accW[nt][i];
  }
  lds_barrier();
  float* sM = sDO;
  if (erase) {
    // ---- dT += dW (diag(beta gam) K^)^T, then M = dT T^T
    if (ccw) {
      v4f acc[NCH];
#pragma unroll
      for (int nt = 0; nt < NCH; ++nt) acc[nt] = z4;
      mm_kk<NCH>(acc, sW + (r0 + l16) * P1, gKn + (int64_t)jb * D, D, D, l16, g4);
#pragma unroll
      for (int nt = 0; nt < NCH; ++nt) {
        const int j = jb + 16 * nt + l16;
        const float bg = sV[lBG * C + j];
#pragma unroll
        for (int i = 0; i < 4; ++i) sY[(r0 + 4 * g4 + i) * P2 + j] += bg * acc[nt][i];
      }
    }
    lds_barrier();  // both halves of each dT row are complete
    if (ccw) {
      v4f acc[NCH];
#pragma unroll
      for (int nt = 0; nt < NCH; ++nt) acc[nt] = z4;
      mm_kk<NCH>(acc, sY + (r0 + l16) * P2, sT + jb * P2, P2, C, l16, g4);
#pragma unroll
      for (int nt = 0; nt < NCH; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) sM[(r0 + 4 * g4 + i) * P2 + jb + 16 * nt + l16] = acc[nt][i];
    }
    lds_barrier();
  }
  // ---- dA = -T^T M -> dKK = beta Gam o dA (strict lower) over dT; dbeta's A
  // term; the dKK Gam terms of dG
  if (ccw) {
    v4f acc[NCH];
#pragma unroll
    for (int nt = 0; nt < NCH; ++nt) acc[nt] = z4;
    if (erase) mm_tn<NCH>(acc, sT + r0 + l16, P2, sM + jb, P2, C, l16, g4);
    float rs[4] = {0.f, 0.f, 0.f, 0.f}, db[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nt = 0; nt < NCH; ++nt) {
      const int j = jb + 16 * nt + l16;
      float cs = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = r0 + 4 * g4 + i;
        float dkk = 0.f;
        if (erase && j < r) {
          const float gda = -expf(sV[lG * C + r] - sV[lG * C + j]) * acc[nt][i];  // Gam o dA
          dkk = sV[lBeta * C + r] * gda;
          db[i] += gKK[r * C + j] * gda;
        }
        sY[r * P2 + j] = dkk;
        const float gg = gKK[r * C + j] * dkk;
        rs[i] += gg;
        cs += gg;
      }
      cs = col4_sum(cs);
      if (g4 == 0) sCol[mt * C + j] += cs;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x = row16_sum(rs[i]), y = row16_sum(db[i]);
      if (l16 == 0) {
        sV[(L::lR + ch) * C + r0 + 4 * g4 + i] += x;
        sV[(L::lDB + ch) * C + r0 + 4 * g4 + i] = y;
      }
    }
  }
  lds_barrier();
  if (rows) {
    // ---- T^T dW -> dK^ += diag(beta gam) T^T dW, and s_r = K^_r . (T^T dW)_r
    if (erase) {
      v4f acc[NH];
#pragma unroll
      for (int nt = 0; nt < NH; ++nt) acc[nt] = z4;
      mm_tn<NH>(acc, sT + r0 + l16, P2, sW + cb, P1, C, l16, g4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = r0 + 4 * g4 + i;
        const float bg = sV[lBG * C + r];
        float sd = 0.f;
#pragma unroll
        for (int nt = 0; nt < NH; ++nt) {
          sd += gKn[r * D + cb + 16 * nt + l16] * acc[nt][i];
          accK[nt][i] += bg * acc[nt][i];
        }
        sd = row16_sum(sd);
        if (l16 == 0) sV[(L::lS + ch) * C + r] = sd;
      }
    }
    // raw q, k rows for the L2-norm backward below, fetched ahead of the
    // last products
    if (direct) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = r0 + 4 * g4 + i;
        const bool in = rr < cr.len;
        const int64_t t = (int64_t)(cr.t0 + rr);
#pragma unroll
        for (int nt = 0; nt < NH; ++nt) {
          const int c = cb + 16 * nt + l16;
          xk[nt][i] = in ? to_f32(kx[t * ks + (int64_t)hq * D + c]) : 0.f;
          xq[nt][i] = in ? to_f32(qx[t * qs + (int64_t)hq * D + c]) : 0.f;
        }
      }
    }
    // ---- dK^ += dQK^T Q^ + (dKK + dKK^T) K^,  dQ^ += dQK K^
    const int r = r0 + l16;
#pragma unroll 2
    for (int k0 = 0; k0 < C; k0 += 4) {
      const int j = k0 + g4;
      const float a1 = sX[j * P2 + r];
      const float a2 = sY[r * P2 + j] + sY[j * P2 + r];
      const float a3 = sX[r * P2 + j];
#pragma unroll
      for (int nt = 0; nt < NH; ++nt) {
        const float qn = gQn[j * D + cb + 16 * nt + l16], kn = gKn[j * D + cb + 16 * nt + l16];
        accK[nt] = mma4(a1, qn, accK[nt]);
        accK[nt] = mma4(a2, kn, accK[nt]);
        accQ[nt] = mma4(a3, kn, accQ[nt]);
      }
    }
    if (!direct) {  // summed over the group's V heads by the QK-head kernel
      float* gdKn = w.cd[mDKn] + bv * C * D;
      float* gdQn = w.cd[mDQn] + bv * C * D;
#pragma unroll
      for (int nt = 0; nt < NH; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t e = (int64_t)(r0 + 4 * g4 + i) * D + cb + 16 * nt + l16;
          gdKn[e] = accK[nt][i];
          gdQn[e] = accQ[nt][i];
        }
    }
  }
  if (direct) {
    // One V head reads this QK head, so dK^ and dQ^ are complete: back through
    // x^ = x / sqrt(|x|^2 + eps) here, dx = r (dx^ - x^ (x^ . dx^)) with
    // r = 1 / sqrt(|x|^2 + eps), the row sums over the NP column parts
    // exchanged through dU's space (dead since the dW store)
    float* sP = sDU;  // [4][NP][C]: |k|^2, k . dK^, |q|^2, q . dQ^
    if (rows) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = r0 + 4 * g4 + i;
        float p0 = 0.f, p1 = 0.f, p2 = 0.f, p3 = 0.f;
#pragma unroll
        for (int nt = 0; nt < NH; ++nt) {
          p0 += xk[nt][i] * xk[nt][i];
          p1 += xk[nt][i] * accK[nt][i];
          p2 += xq[nt][i] * xq[nt][i];
          p3 += xq[nt][i] * accQ[nt][i];
        }
        p0 = row16_sum(p0);
        p1 = row16_sum(p1);
        p2 = row16_sum(p2);
        p3 = row16_sum(p3);
        if (l16 == 0) {
          sP[(0 * NP + ch) * C + r] = p0;
          sP[(1 * NP + ch) * C + r] = p1;
          sP[(2 * NP + ch) * C + r] = p2;
          sP[(3 * NP + ch) * C + r] = p3;
        }
      }
    }
    lds_barrier();
    if (rows) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = r0 + 4 * g4 + i;
        if (r >= cr.len) continue;
        const int64_t t = (int64_t)(cr.t0 + r);
        float sk = 0.f, dkx = 0.f, sq = 0.f, dqx = 0.f;
#pragma unroll
        for (int q = 0; q < NP; ++q) {
          sk += sP[(0 * NP + q) * C + r];
          dkx += sP[(1 * NP + q) * C + r];
          sq += sP[(2 * NP + q) * C + r];
          dqx += sP[(3 * NP + q) * C + r];
        }
        const float rk = l2norm ? 1.0f / sqrtf(sk + 1e-6f) : 1.f, rq = l2norm ? 1.0f / sqrtf(sq + 1e-6f) : 1.f;
        const float ck = l2norm ? dkx * rk * rk * rk : 0.f, cq = l2norm ? dqx * rq * rq * rq : 0.f;
#pragma unroll
        for (int nt = 0; nt < NH; ++nt) {
          const int c = cb + 16 * nt + l16;
          dk[t * dks + (int64_t)hq * D + c] = from_f32<T>(accK[nt][i] * rk - xk[nt][i] * ck);
          dq[t * dqs + (int64_t)hq * D + c] = from_f32<T>(accQ[nt][i] * rq - xq[nt][i] * cq);
        }
      }
    }
  }
  lds_barrier();
  // ---- dG per row, its reverse cumulative sum dg (a suffix scan over the
  // lanes of wave 0, lane r holding row r), and dbeta
  if (wave == 0) {
    const int r = lane;
    const bool on = r < C;
    float col = 0.f, d = 0.f, u = 0.f, db = 0.f;
    if (on) {
      for (int q = 0; q < NC; ++q) col += sCol[q * C + r];
      float a = 0.f, sd = 0.f, rw = 0.f;
#pragma unroll
      for (int q = 0; q < NP; ++q) {
        a += sV[(L::lA + q) * C + r];
        sd += sV[(L::lS + q) * C + r];
        rw += sV[(L::lR + q) * C + r];
        db += sV[(L::lB + q) * C + r] + sV[(L::lDB + q) * C + r];
      }
      u = sV[lU * C + r];
      d = sV[lSG * C + r] * a + sV[lBG * C + r] * sd + rw - col - u;
      if (erase) db += sV[lGam * C + r] * sd;
    }
    const float us = wave_sum(u);
    float xd = 0.f;
#pragma unroll
    for (int q = 0; q < 4 * NP; ++q) xd += sRed[q];
    if (r == C - 1) d += us + sV[lGam * C + r] * xd;
#pragma unroll
    for (int off = 1; off < 64; off *= 2) {
      const float t = __shfl_down(d, off, 64);
      if (r + off < 64) d += t;
    }
    if (r < cr.len) {
      const int64_t t = (int64_t)(cr.t0 + r);
      dg[t * h_v + h] = d;
      dbeta[t * h_v + h] = db;
    }
  }
}

// Column parts per row tile: 4 (16 waves, 4 per SIMD at one workgroup per CU)
constexpr int kLocalParts = 4;

template <typename T, int D, int C>
hipError_t launch_local(const BwdWs& w, const PrefillBwdParams& p, int64_t ncm, hipStream_t stream) {
  constexpr int NP = kLocalParts;
  const size_t lds = (size_t)LocalLayout<D, C, NP>::floats * sizeof(float);
  const void* f = reinterpret_cast<const void*>(bwd_local_kernel<T, D, C, NP>);
  hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_local_kernel<T, D, C, NP>), dim3((unsigned)(ncm * p.h_v)), dim3(256 * NP), lds, stream, w,
                     static_cast<const T*>(p.v), p.v_stride, static_cast<T*>(p.dv), p.dv_stride, p.dg, p.dbeta,
                     p.h_qk, p.h_v, p.scale, p.erase, static_cast<const T*>(p.q), static_cast<const T*>(p.k),
                     p.q_stride, p.k_stride, static_cast<T*>(p.dq), static_cast<T*>(p.dk), p.dq_stride, p.dk_stride,
                     p.l2norm, p.h_v == p.h_qk);
  return hipGetLastError();
}

// -------------------------------------------------------- final, QK head
// Per (token, QK head): sum dK^ and dQ^ over the V heads of the group, then
// back through x^ = x / sqrt(|x|^2 + eps): dx = dx^/n - x (x.dx^)/n^3.
template <typename T>
__global__ __launch_bounds__(64) void bwd_final_qk_kernel(BwdWs w, const int32_t* cu, int n_seqs, const T* q,
                                                          const T* k, int64_t qs, int64_t ks, T* dq, T* dk,
                                                          int64_t dqs, int64_t dks, int h_qk, int h_v, int D,
                                                          int C, int l2norm) {
  const int64_t t = blockIdx.x;
  const int hq = blockIdx.y, lane = threadIdx.x, grp = h_v / h_qk;
  const int n = cu ? seq_index(cu, n_seqs, t) : 0;
  const int64_t s = cu ? cu[n] : 0;
  const int gc = w.co[n] + (int)((t - s) / C), r = (int)((t - s) % C);
  // lane l holds elements D/64 l .. of the row (one 4- or 8-byte access each)
  const int per = D / 64, c0 = per * lane;
  for (int which = 0; which < 2; ++which) {
    const float* src = which ? w.cd[mDQn] : w.cd[mDKn];
    const T* xs = (which ? q : k) + t * (which ? qs : ks) + (int64_t)hq * D + c0;
    float d[2] = {0.f, 0.f}, x[2] = {0.f, 0.f};
    for (int j = 0; j < grp; ++j) {
      const float* sr = src + (((int64_t)gc * h_v + hq * grp + j) * C + r) * D + c0;
      if (per == 2) {
        const float2 f = *reinterpret_cast<const float2*>(sr);
        d[0] += f.x;
        d[1] += f.y;
      } else {
        d[0] += sr[0];
      }
    }
    if (per == 2) load2(xs, x[0], x[1]);
    else x[0] = to_f32(xs[0]);
    if (l2norm) {
      const float ss = wave_sum(x[0] * x[0] + x[1] * x[1]), xd = wave_sum(x[0] * d[0] + x[1] * d[1]);
      const float rn = 1.0f / sqrtf(ss + 1e-6f);
      for (int i = 0; i < 2; ++i) d[i] = d[i] * rn - x[i] * xd * rn * rn * rn;
    }
    T* dst = (which ? dq : dk) + t * (which ? dqs : dks) + (int64_t)hq * D + c0;
    if (per == 2) {
      const T o[2] = {from_f32<T>(d[0]), from_f32<T>(d[1])};
      __builtin_memcpy(dst, o, sizeof(o));
    } else {
      dst[0] = from_f32<T>(d[0]);
    }
  }
}

// ------------------------------------------------------------ conv backward
// z = sum_j w_j xp[t + j] (+ b) over the padded history xp = (state ++ x) of
// the token's sequence, y = act(z), dz = dy act'(z).

__device__ inline void seq_of(const int32_t* cu, int n_seqs, int64_t T, int64_t t, int& n, int64_t& s,
                              int64_t& e) {
  n = cu ? seq_index(cu, n_seqs, t) : 0;
  s = cu ? cu[n] : 0;
  e = cu ? cu[n + 1] : T;
}

template <typename T>
__device__ inline float conv_xp(const T* x, const T* state, int64_t s, int n, int C, int W, int c, int64_t i) {
  // padded-history entry i of sequence n (starting at token s), channel c
  if (i < W - 1) return state ? to_f32(state[((int64_t)n * C + c) * (W - 1) + i]) : 0.f;
  return to_f32(x[(s + i - (W - 1)) * C + c]);
}

template <typename T>
__device__ inline float conv_dz(const T* x, const T* w, const T* bias, const T* state, const T* dy, int64_t s,
                                int n, int C, int W, int c, int64_t u, int act) {
  // gradient at pre-activation z of local token u of sequence n
  float z = bias ? to_f32(bias[c]) : 0.f;
  for (int j = 0; j < W; ++j) z = fmaf(to_f32(w[c * W + j]), conv_xp(x, state, s, n, C, W, c, u + j), z);
  const float d = to_f32(dy[(s + u) * C + c]);
  if (!act) return d;
  const float sg = 1.0f / (1.0f + expf(-z));
  return d * sg * (1.0f + z * (1.0f - sg));
}

// One pass per (token tile, 8 channels): each thread walks the tile plus the
// W-1 tokens after it, computing every dz once.  dz_tau adds w_{W-1-k} dz_tau
// to the pending dx of token tau - k (k < W, same sequence); a token's dx is
// complete once tau has moved W-1 past it, or at its sequence's end, where
// the gradient of the new conv state adds onto the last W-1 tokens.  The
// weight and bias partial sums of the tile's own tokens go to the workspace.
constexpr int kConvBT = 32;

// 8 consecutive elements as raw bits (16 B of bf16, 32 B of fp32), so that
// loads can run ahead of the arithmetic that widens them
template <typename T> struct Row8;
template <> struct Row8<__bf16> {
  uint4 a;
  __device__ __forceinline__ void load(const __bf16* p) { a = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void get(float (&v)[8]) const {
    v[0] = bf16_lo(a.x); v[1] = bf16_hi(a.x); v[2] = bf16_lo(a.y); v[3] = bf16_hi(a.y);
    v[4] = bf16_lo(a.z); v[5] = bf16_hi(a.z); v[6] = bf16_lo(a.w); v[7] = bf16_hi(a.w);
  }
};
template <> struct Row8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = reinterpret_cast<const float4*>(p)[0];
    b = reinterpret_cast<const float4*>(p)[1];
  }
  __device__ __forceinline__ void get(float (&v)[8]) const {
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
};

template <typename T, int W>
__global__ __launch_bounds__(256) void conv_bwd_kernel(const T* x, const T* w, const T* bias, const T* state,
                                                       const T* dy, const float* dns, const int32_t* cu,
                                                       int n_seqs, int64_t Tt, int C, int act, T* dx,
                                                       float* part) {
  const int c0 = (blockIdx.y * 256 + threadIdx.x) * 8;
  if (c0 >= C) return;
  const int64_t t0 = (int64_t)blockIdx.x * kConvBT, t1 = min(t0 + kConvBT, Tt), tend = min(t1 + W - 1, Tt);
  float wt[W][8], bs[8], xw[W][8], pend[W][8], aw[W + 1][8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int j = 0; j < W; ++j) {
      wt[j][i] = to_f32(w[(c0 + i) * W + j]);
      aw[j][i] = 0.f;
    }
    aw[W][i] = 0.f;
    bs[i] = bias ? to_f32(bias[c0 + i]) : 0.f;
  }
  int n = 0;
  int64_t s = 0, e = 0;
  // x and dy rows two tokens ahead
  Row8<T> px[2], pd[2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
    if (t0 + u < tend) {
      px[u].load(x + (t0 + u) * C + c0);
      pd[u].load(dy + (t0 + u) * C + c0);
    }
  for (int64_t tau = t0; tau < tend; ++tau) {
    float d8[8];
    px[0].get(xw[W - 1]);
    pd[0].get(d8);
    px[0] = px[1];
    pd[0] = pd[1];
    if (tau + 2 < tend) {
      px[1].load(x + (tau + 2) * C + c0);
      pd[1].load(dy + (tau + 2) * C + c0);
    }
    if (tau == t0 || tau >= e) {
      seq_of(cu, n_seqs, Tt, tau, n, s, e);
#pragma unroll
      for (int j = 0; j < W - 1; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) xw[j][i] = conv_xp(x, state, s, n, C, W, c0 + i, tau - s + j);
#pragma unroll
      for (int k = 0; k < W; ++k)
#pragma unroll
        for (int i = 0; i < 8; ++i) pend[k][i] = 0.f;
    }
    float dz[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float z = bs[i];
#pragma unroll
      for (int j = 0; j < W; ++j) z = fmaf(wt[j][i], xw[j][i], z);
      if (act) {
        const float sg = 1.0f / (1.0f + expf(-z));
        dz[i] = d8[i] * sg * (1.0f + z * (1.0f - sg));
      } else {
        dz[i] = d8[i];
      }
    }
    if (tau < t1) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int j = 0; j < W; ++j) aw[j][i] = fmaf(dz[i], xw[j][i], aw[j][i]);
        aw[W][i] += dz[i];
      }
    }
#pragma unroll
    for (int k = W - 1; k > 0; --k)
#pragma unroll
      for (int i = 0; i < 8; ++i) pend[k][i] = pend[k - 1][i];
#pragma unroll
    for (int i = 0; i < 8; ++i) pend[0][i] = 0.f;
#pragma unroll
    for (int k = 0; k < W; ++k)
      if (tau - k >= s)
#pragma unroll
        for (int i = 0; i < 8; ++i) pend[k][i] = fmaf(wt[W - 1 - k][i], dz[i], pend[k][i]);
    const int64_t td = tau - (W - 1);
    if (td >= s && td >= t0 && td < t1) store8(dx + td * C + c0, pend[W - 1]);
    if (tau == e - 1) {
      const int64_t L = e - s;
#pragma unroll
      for (int k = 0; k < W - 1; ++k) {
        const int64_t t = tau - k;
        if (t >= s && t >= t0 && t < t1) {
          const int64_t ip = t - s + W - 1;
          float v[8];
#pragma unroll
          for (int i = 0; i < 8; ++i)
            v[i] = pend[k][i] + ((dns && ip >= L) ? dns[((int64_t)n * C + c0 + i) * (W - 1) + (ip - L)] : 0.f);
          store8(dx + t * C + c0, v);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < W - 1; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) xw[j][i] = xw[j + 1][i];
  }
  float* pp = part + (int64_t)blockIdx.x * 5 * C + c0;
#pragma unroll
  for (int j = 0; j < W; ++j) store8(pp + (int64_t)j * C, aw[j]);
  store8(pp + (int64_t)4 * C, aw[W]);
}

template <typename T>
__global__ __launch_bounds__(256) void conv_bwd_state_kernel(const T* x, const T* w, const T* bias, const T* state,
                                                             const T* dy, const float* dns, const int32_t* cu,
                                                             int n_seqs, int64_t Tt, int C, int W, int act,
                                                             float* dstate) {
  const int c = blockIdx.y * 256 + threadIdx.x, n = blockIdx.x;
  if (c >= C) return;
  const int64_t s = cu ? cu[n] : 0, L = (cu ? cu[n + 1] : Tt) - s;
  for (int i = 0; i < W - 1; ++i) {
    float acc = 0.f;
    for (int j = 0; j < W; ++j) {
      const int64_t u = i - j;
      if (u >= 0 && u < L) acc = fmaf(to_f32(w[c * W + j]), conv_dz(x, w, bias, state, dy, s, n, C, W, c, u, act), acc);
    }
    if (dns && i >= L) acc += dns[((int64_t)n * C + c) * (W - 1) + (i - L)];
    dstate[((int64_t)n * C + c) * (W - 1) + i] = acc;
  }
}

// Per 64 channels: four thread groups each sum every fourth tile, then the
// four partial sums are added in a fixed order (deterministic results).
__global__ __launch_bounds__(256) void conv_bwd_reduce_kernel(const float* part, int ntiles, int C, int W,
                                                              float* dweight, float* dbias) {
  __shared__ float red[4][5][64];
  const int cl = threadIdx.x & 63, grp = threadIdx.x >> 6, c = blockIdx.x * 64 + cl;
  float acc[5] = {0.f, 0.f, 0.f, 0.f, 0.f};
  if (c < C)
    for (int t = grp; t < ntiles; t += 4)
#pragma unroll
      for (int j = 0; j < 5; ++j) acc[j] += part[((int64_t)t * 5 + j) * C + c];
#pragma unroll
  for (int j = 0; j < 5; ++j) red[grp][j][cl] = acc[j];
  __syncthreads();
  if (grp == 0 && c < C) {
    for (int j = 0; j < 5; ++j) acc[j] = ((red[0][j][cl] + red[1][j][cl]) + red[2][j][cl]) + red[3][j][cl];
    for (int j = 0; j < W; ++j) dweight[c * W + j] = acc[j];
    if (dbias) dbias[c] = acc[4];
  }
}

// ------------------------------------------------------------------ host
struct Launcher {
  hipStream_t st;
  hipError_t err = hipSuccess;
  void check() {
    if (err == hipSuccess) err = hipGetLastError();
  }
};

BG gemm(const float* A, const float* B, float* Cm, int M, int N, int K, int lda, int ldb, int ldc, int ta, int tb,
        int64_t a_sc, int64_t a_sh, int a_hdiv, int64_t b_sc, int64_t b_sh, int b_hdiv, int64_t c_sc, int64_t c_sh,
        int H, float alpha, int accum, const int* nc) {
  return BG{A, B, Cm, M, N, K, lda, ldb, ldc, a_sc, a_sh, b_sc, b_sh, c_sc, c_sh, a_hdiv, b_hdiv, H, ta, tb,
            accum, alpha, nc, nullptr, nullptr, 0};
}

void run_gemm(Launcher& L, const BG& p, int64_t ncm) {
  if (L.err != hipSuccess) return;
  const dim3 grid((unsigned)(ncm * p.H), (unsigned)(((p.M + 63) / 64) * ((p.N + 63) / 64)));
  hipLaunchKernelGGL(bgemm_kernel, grid, dim3(256), 0, L.st, p);
  L.check();
}

template <typename T>
hipError_t prefill_backward_impl(const PrefillBwdParams& p, int D, hipStream_t stream) {
  const int C = p.chunk, hq = p.h_qk, hv = p.h_v, grp = hv / hq;
  const BwdSizes sz = bwd_sizes(p.total_tokens, p.n_seqs, hq, hv, D, C);
  const int64_t ncm = sz.ncm;
  BwdWs w = bwd_carve(p.workspace, p.total_tokens, p.n_seqs, hq, hv, D, C);
  Launcher L{stream};
  hipLaunchKernelGGL(bwd_plan_kernel, dim3(1), dim3(256), 0, stream, w, p.cu_seqlens, p.n_seqs, p.total_tokens, C,
                     ncm);
  L.check();
  const T* q = static_cast<const T*>(p.q);
  const T* k = static_cast<const T*>(p.k);
  const T* v = static_cast<const T*>(p.v);
  if (p.total_tokens > 0) {
    hipLaunchKernelGGL(bwd_stage_qk_kernel<T>, dim3((unsigned)(ncm * hq)), dim3(256), 0, stream, w, q, k,
                       p.q_stride, p.k_stride, hq, D, C, p.l2norm);
    L.check();
  }
  const int64_t CC = (int64_t)C * C, CD = (int64_t)C * D, DD = (int64_t)D * D;
  const int* nc = w.nc;
  // Gram matrices per QK head: KK = Kn Kn^T, QK = Qn Kn^T
  run_gemm(L, gemm(w.Kn, w.Kn, w.KK, C, C, D, D, D, C, 0, 1, hq * CD, CD, 1, hq * CD, CD, 1, hq * CC, CC, hq, 1.f, 0, nc), ncm);
  run_gemm(L, gemm(w.Qn, w.Kn, w.QK, C, C, D, D, D, C, 0, 1, hq * CD, CD, 1, hq * CD, CD, 1, hq * CC, CC, hq, 1.f, 0, nc), ncm);
  if (L.err != hipSuccess) return L.err;
  if (p.total_tokens > 0) {
    hipLaunchKernelGGL(bwd_prep_kernel<T>, dim3((unsigned)(ncm * hv)), dim3(256), 0, stream, w, p.g, p.beta, v,
                       p.v_stride, static_cast<const T*>(p.d_o), hq, hv, D, C, p.scale, p.erase);
    L.check();
  }
  // per V head (stride hv * size per chunk, size per head)
  auto VH = [&](float* A, float* B, float* Cm, int M, int N, int K, int lda, int ldb, int ldc, int ta, int tb,
                int64_t sa, int64_t sb, int64_t sc, float alpha, int accum, int b_hdiv = 1, int64_t b_chunk = -1) {
    const int64_t bsc = b_chunk < 0 ? hv * sb : b_chunk;
    run_gemm(L, gemm(A, B, Cm, M, N, K, lda, ldb, ldc, ta, tb, hv * sa, sa, 1, bsc, sb, b_hdiv, hv * sc, sc, hv,
                     alpha, accum, nc),
             ncm);
  };
  float** cc = w.cc;
  float** cd = w.cd;
  float** dd = w.dd;
  // W = T diag(beta gam) K^ (rows of K^ scaled as they are read), Ut = T BV
  {
    BG g = gemm(cc[cT], w.Kn, cd[mW], C, D, C, C, D, D, 0, 0, hv * CC, CC, 1, hq * CD, CD, grp, hv * CD, CD, hv,
                1.f, 0, nc);
    g.bs = w.vec + kVecBG * C;
    g.vstr = kNVec * C;
    run_gemm(L, g, ncm);
  }
  VH(cc[cT], cd[mBV], cd[mUt], C, D, C, C, D, D, 0, 0, CC, CD, CD, 1.f, 0);
  if (L.err != hipSuccess) return L.err;
  // PdO = Pm^T dO and Z (the reverse chain's inputs)
  VH(cc[cPm], cd[mDO], cd[mPdO], C, D, C, C, D, D, 1, 0, CC, CD, CD, 1.f, 0);
  {  // Z = (scale diag(gam) Q^)^T dO
    BG g = gemm(w.Qn, cd[mDO], dd[xZ], D, D, C, D, D, D, 1, 0, hq * CD, CD, grp, hv * CD, CD, 1, hv * DD, DD, hv,
                1.f, 0, nc);
    g.as = w.vec + kVecSG * C;
    g.vstr = kNVec * C;
    run_gemm(L, g, ncm);
  }
  if (L.err != hipSuccess) return L.err;
  {
    hipError_t e;
    if constexpr (std::is_same<T, __bf16>::value) {
      if (D == 64)
        e = C == 16 ? launch_chains_bf16<64, 16>(w, p, stream) : C == 32 ? launch_chains_bf16<64, 32>(w, p, stream)
                                                               : launch_chains_bf16<64, 64>(w, p, stream);
      else
        e = C == 16 ? launch_chains_bf16<128, 16>(w, p, stream)
                    : C == 32 ? launch_chains_bf16<128, 32>(w, p, stream) : launch_chains_bf16<128, 64>(w, p, stream);
    } else {
      if (D == 64)
        e = C == 16 ? launch_chains<64, 16>(w, p, stream) : C == 32 ? launch_chains<64, 32>(w, p, stream)
                                                            : launch_chains<64, 64>(w, p, stream);
      else
        e = C == 16 ? launch_chains<128, 16>(w, p, stream) : C == 32 ? launch_chains<128, 32>(w, p, stream)
                                                             : launch_chains<128, 64>(w, p, stream);
    }
    if (e != hipSuccess) return e;
  }
  // every chunk-local gradient, one workgroup per (chunk, V head)
  if (p.total_tokens > 0) {
    hipError_t e;
    if (D == 64)
      e = C == 16 ? launch_local<T, 64, 16>(w, p, ncm, stream)
                  : C == 32 ? launch_local<T, 64, 32>(w, p, ncm, stream) : launch_local<T, 64, 64>(w, p, ncm, stream);
    else
      e = C == 16 ? launch_local<T, 128, 16>(w, p, ncm, stream)
                  : C == 32 ? launch_local<T, 128, 32>(w, p, ncm, stream) : launch_local<T, 128, 64>(w, p, ncm, stream);
    if (e != hipSuccess) return e;
    // with one V head per QK head the fused kernel has written dq and dk
    if (hv != hq) {
      hipLaunchKernelGGL(bwd_final_qk_kernel<T>, dim3((unsigned)p.total_tokens, (unsigned)hq), dim3(64), 0, stream, w,
                         p.cu_seqlens, p.n_seqs, q, k, p.q_stride, p.k_stride, static_cast<T*>(p.dq),
                         static_cast<T*>(p.dk), p.dq_stride, p.dk_stride, hq, hv, D, C, p.l2norm);
      L.check();
    }
  }
  return L.err;
}

template <typename T>
hipError_t conv_backward_impl(const ConvBwdParams& p, hipStream_t stream) {
  const T* x = static_cast<const T*>(p.x);
  const T* w = static_cast<const T*>(p.weight);
  const T* b = static_cast<const T*>(p.bias);
  const T* st = static_cast<const T*>(p.conv_state);
  const T* dy = static_cast<const T*>(p.dy);
  const int cg = (p.channels + 255) / 256;
  const int cg8 = (p.channels / 8 + 255) / 256;
  const int ntiles = (int)((p.total_tokens + kConvBT - 1) / kConvBT);
  float* part = static_cast<float*>(p.workspace);
  if (ntiles > 0) {
    const dim3 grid(ntiles, cg8);
    T* dx = static_cast<T*>(p.dx);
    if (p.width == 4)
      hipLaunchKernelGGL((conv_bwd_kernel<T, 4>), grid, dim3(256), 0, stream, x, w, b, st, dy, p.d_new_state,
                         p.cu_seqlens, p.n_seqs, p.total_tokens, p.channels, p.act, dx, part);
    else if (p.width == 3)
      hipLaunchKernelGGL((conv_bwd_kernel<T, 3>), grid, dim3(256), 0, stream, x, w, b, st, dy, p.d_new_state,
                         p.cu_seqlens, p.n_seqs, p.total_tokens, p.channels, p.act, dx, part);
    else
      hipLaunchKernelGGL((conv_bwd_kernel<T, 2>), grid, dim3(256), 0, stream, x, w, b, st, dy, p.d_new_state,
                         p.cu_seqlens, p.n_seqs, p.total_tokens, p.channels, p.act, dx, part);
  }
  hipLaunchKernelGGL(conv_bwd_reduce_kernel, dim3((p.channels + 63) / 64), dim3(256), 0, stream, part, ntiles,
                     p.channels, p.width, p.dweight, p.dbias);
  if (p.d_conv_state)
    hipLaunchKernelGGL(conv_bwd_state_kernel<T>, dim3(p.n_seqs, cg), dim3(256), 0, stream, x, w, b, st, dy,
                       p.d_new_state, p.cu_seqlens, p.n_seqs, p.total_tokens, p.channels, p.width, p.act,
                       p.d_conv_state);
  return hipGetLastError();
}

// ------------------------------------------------------------- windows
// The workspace above holds every chunk of the call (2.6 GB for the 9B
// layer, 27 GB for the 27B one).  For one sequence whose workspace would pass
// kBwdBudget the call runs in windows of wt tokens (a multiple of the chunk):
//   1. a forward pass over the windows in order (gdn_prefill's own kernels,
//      o into scratch) leaves the state at every window start;
//   2. the backward above runs on each window from the last to the first,
//      starting from that window's state, with the state gradient of the
//      window after it as its final-state gradient; the initial-state
//      gradient it returns is the next (earlier) window's.
// Every token's gradients come from one window, so nothing is accumulated.
// The workspace then holds one window's backward, the forward's workspace
// and o for one window, the window-start states and two state gradients.
constexpr size_t kBwdBudgetDefault = (size_t)4 << 30;

size_t bwd_budget() {
  const char* e = std::getenv("GDN_BWD_BUDGET_MB");  // tuning and tests: a smaller budget
  const long long mb = e ? std::atoll(e) : 0;
  return mb > 0 ? (size_t)mb << 20 : kBwdBudgetDefault;
}

struct BwdWindows {
  bool on;
  int64_t wt;
  int nwin;
  size_t o_fwd, o_o, o_ck, o_cy, total;
};

BwdWindows bwd_windows(int io_dtype, int64_t T, int n_seqs, int h_qk, int h_v, int D, int C) {
  BwdWindows w{false, T, 1, 0, 0, 0, 0, bwd_sizes(T, n_seqs, h_qk, h_v, D, C).total};
  const size_t budget = bwd_budget();
  if (n_seqs != 1 || w.total <= budget || T <= C) return w;
  const size_t hs = (size_t)h_v * D * D * 4, es = io_dtype == 1 ? 2 : 4;
  auto layout = [&](int64_t wt) {
    BwdWindows x{true, wt, (int)((T + wt - 1) / wt), 0, 0, 0, 0, 0};
    x.o_fwd = bwd_sizes(wt, 1, h_qk, h_v, D, C).total;
    x.o_o = x.o_fwd + a256(prefill_workspace_bytes(io_dtype, wt, 1, h_v, D, C, 0));
    x.o_ck = x.o_o + a256((size_t)wt * h_v * D * es);
    x.o_cy = x.o_ck + a256((size_t)x.nwin * hs);
    x.total = x.o_cy + 2 * a256(hs);
    return x;
  };
  int64_t wt = (T + C - 1) / C * C;
  BwdWindows x = layout(wt);
  while (x.total > budget && wt > C) {
    wt = ((wt / 2) + C - 1) / C * C;
    x = layout(wt);
  }
  return x;
}

template <typename T>
hipError_t prefill_backward_windows(const PrefillBwdParams& p, int D, const BwdWindows& bw, hipStream_t stream) {
  unsigned char* ws = static_cast<unsigned char*>(p.workspace);
  const size_t hs = (size_t)p.h_v * D * D;
  float* ck = reinterpret_cast<float*>(ws + bw.o_ck);  // [nwin][h_v][D][D]: state at each window start
  float* cy[2] = {reinterpret_cast<float*>(ws + bw.o_cy), reinterpret_cast<float*>(ws + bw.o_cy + a256(hs * 4))};
  const int64_t ntok = p.total_tokens;
  auto span = [&](int w, int64_t& t0, int64_t& n) {
    t0 = (int64_t)w * bw.wt;
    n = std::min(bw.wt, ntok - t0);
  };
  // 1. forward over the windows in order: the state at every window start
  for (int w = 0; w + 1 < bw.nwin; ++w) {
    int64_t t0, n;
    span(w, t0, n);
    PrefillParams f{static_cast<const T*>(p.q) + t0 * p.q_stride, static_cast<const T*>(p.k) + t0 * p.k_stride,
                    static_cast<const T*>(p.v) + t0 * p.v_stride, p.q_stride, p.k_stride, p.v_stride,
                    p.g + t0 * p.h_v, p.beta + t0 * p.h_v,
                    w == 0 ? static_cast<const void*>(p.initial_state) : static_cast<const void*>(ck + w * hs),
                    ck + (w + 1) * hs, ws + bw.o_o, nullptr, n, 1, p.h_qk, p.h_v, p.chunk, p.l2norm, p.scale,
                    ws + bw.o_fwd, bw.o_o - bw.o_fwd, p.erase, 0, nullptr, nullptr, 0};
    const hipError_t e = launch_prefill(f, std::is_same<T, __bf16>::value ? 1 : 0, D, stream);
    if (e != hipSuccess) return e;
  }
  // 2. the backward of each window, last to first
  for (int w = bw.nwin - 1; w >= 0; --w) {
    int64_t t0, n;
    span(w, t0, n);
    PrefillBwdParams b = p;
    b.q = static_cast<const T*>(p.q) + t0 * p.q_stride;
    b.k = static_cast<const T*>(p.k) + t0 * p.k_stride;
    b.v = static_cast<const T*>(p.v) + t0 * p.v_stride;
    b.g = p.g + t0 * p.h_v;
    b.beta = p.beta + t0 * p.h_v;
    b.initial_state = w == 0 ? p.initial_state : ck + w * hs;
    b.d_o = static_cast<const T*>(p.d_o) + t0 * p.h_v * D;
    b.d_final_state = w == bw.nwin - 1 ? p.d_final_state : cy[(w + 1) & 1];
    b.dq = static_cast<T*>(p.dq) + t0 * p.dq_stride;
    b.dk = static_cast<T*>(p.dk) + t0 * p.dk_stride;
    b.dv = static_cast<T*>(p.dv) + t0 * p.dv_stride;
    b.dg = p.dg + t0 * p.h_v;
    b.dbeta = p.dbeta + t0 * p.h_v;
    b.d_initial_state = w == 0 ? p.d_initial_state : cy[w & 1];
    b.total_tokens = n;
    b.workspace = ws;
    const hipError_t e = prefill_backward_impl<T>(b, D, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// ------------------------------------------------------- packs, serially
// A pack whose whole-call workspace would pass the budget runs its sequences
// one after another, each as one sequence (in windows when it is long), in
// one workspace sized for the worst case: every token in one sequence, and at
// least the budget (a shorter sequence may run whole within it).  The
// sequence offsets are read back first, which synchronises the stream once,
// so such a call is refused under stream capture.
bool pack_serial(int64_t T, int n_seqs, int h_qk, int h_v, int D, int C) {
  return n_seqs > 1 && bwd_sizes(T, n_seqs, h_qk, h_v, D, C).total > bwd_budget();
}
size_t pack_serial_bytes(int io_dtype, int64_t T, int h_qk, int h_v, int D, int C) {
  return a256(std::max(bwd_budget(), bwd_windows(io_dtype, T, 1, h_qk, h_v, D, C).total));
}

}  // namespace

size_t prefill_backward_workspace_bytes(int io_dtype, int64_t total_tokens, int n_seqs, int h_qk, int h_v, int d,
                                        int chunk) {
  if (pack_serial(total_tokens, n_seqs, h_qk, h_v, d, chunk))
    return pack_serial_bytes(io_dtype, total_tokens, h_qk, h_v, d, chunk);
  return bwd_windows(io_dtype, total_tokens, n_seqs, h_qk, h_v, d, chunk).total;
}

template <typename T>
hipError_t prefill_backward_pack(const PrefillBwdParams& p, int io_dtype, int D, hipStream_t stream) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(stream, &cs);
  if (e != hipSuccess) return e;
  if (cs != hipStreamCaptureStatusNone) return hipErrorStreamCaptureUnsupported;
  std::vector<int32_t> cu((size_t)p.n_seqs + 1);
  e = hipMemcpyAsync(cu.data(), p.cu_seqlens, cu.size() * sizeof(int32_t), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return e;
  const size_t hs = (size_t)p.h_v * D * D;
  for (int n = 0; n < p.n_seqs; ++n) {
    const int64_t t0 = cu[n], len = (int64_t)cu[n + 1] - cu[n];
    if (t0 < 0 || len < 0 || t0 + len > p.total_tokens) return hipErrorInvalidValue;
    PrefillBwdParams b = p;
    b.q = static_cast<const T*>(p.q) + t0 * p.q_stride;
    b.k = static_cast<const T*>(p.k) + t0 * p.k_stride;
    b.v = static_cast<const T*>(p.v) + t0 * p.v_stride;
    b.g = p.g + t0 * p.h_v;
    b.beta = p.beta + t0 * p.h_v;
    b.d_o = static_cast<const T*>(p.d_o) + t0 * p.h_v * D;
    b.dq = static_cast<T*>(p.dq) + t0 * p.dq_stride;
    b.dk = static_cast<T*>(p.dk) + t0 * p.dk_stride;
    b.dv = static_cast<T*>(p.dv) + t0 * p.dv_stride;
    b.dg = p.dg + t0 * p.h_v;
    b.dbeta = p.dbeta + t0 * p.h_v;
    b.initial_state = p.initial_state ? p.initial_state + n * hs : nullptr;
    b.d_final_state = p.d_final_state ? p.d_final_state + n * hs : nullptr;
    b.d_initial_state = p.d_initial_state ? p.d_initial_state + n * hs : nullptr;
    b.cu_seqlens = nullptr;
    b.n_seqs = 1;
    b.total_tokens = len;
    e = launch_prefill_backward(b, io_dtype, D, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_prefill_backward(const PrefillBwdParams& p, int io_dtype, int d, hipStream_t stream) {
  if (pack_serial(p.total_tokens, p.n_seqs, p.h_qk, p.h_v, d, p.chunk))
    return io_dtype == 1 ? prefill_backward_pack<__bf16>(p, io_dtype, d, stream)
                         : prefill_backward_pack<float>(p, io_dtype, d, stream);
  const BwdWindows bw = bwd_windows(io_dtype, p.total_tokens, p.n_seqs, p.h_qk, p.h_v, d, p.chunk);
  if (bw.on)
    return io_dtype == 1 ? prefill_backward_windows<__bf16>(p, d, bw, stream)
                         : prefill_backward_windows<float>(p, d, bw, stream);
  return io_dtype == 1 ? prefill_backward_impl<__bf16>(p, d, stream) : prefill_backward_impl<float>(p, d, stream);
}

size_t conv1d_backward_workspace_bytes(int64_t total_tokens, int channels) {
  const int64_t ntiles = (total_tokens + kConvBT - 1) / kConvBT;
  return a256((size_t)(ntiles > 0 ? ntiles : 1) * channels * 5 * sizeof(float));
}

hipError_t launch_conv1d_backward(const ConvBwdParams& p, int dtype, hipStream_t stream) {
  return dtype == 1 ? conv_backward_impl<__bf16>(p, stream) : conv_backward_impl<float>(p, stream);
}

}  // namespace gdn
