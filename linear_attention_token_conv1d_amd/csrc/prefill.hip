// gdn_prefill: chunked gated delta rule on gfx950.
//
// Math (per sequence, V head; within a chunk of L <= C tokens, G_r the
// inclusive cumulative sum of g, gamma_r = e^{G_r}, e_r = e^{G_{L-1} - G_r},
// k^_r = rk_r k_r and q^_r = rq_r q_r the L2-normalised rows):
//   A_rj  = beta_r e^{G_r - G_j} (k^_r . k^_j)            j <  r   (strict lower)
//   T     = (I + A)^-1,   Tb = T diag(beta)
//   P_rj  = scale e^{G_r - G_j} (q^_r . k^_j)              j <= r
//   X1    = K S^T,  Y = Q S^T                   (raw K, Q rows)
//   R     = V - diag(gamma rk) X1
//   U     = Tb R                                (the chunk's delta writes)
//   O     = diag(scale gamma rq) Y + P U
//   S^T  <- gamma_{L-1} S^T + K^T diag(e rk) U
// This is the recurrence S_t = a_t S_{t-1}(I - b_t k_t k_t^T) + b_t v_t k_t^T,
// o_t = scale S_t q_t ("Inside Qwen3.5", sections 4-5) unrolled over a chunk;
// only e^{x} with x <= 0 is ever formed.
//
// Work split: one workgroup per (sequence, V head, block of 64 d_v columns),
// 4 waves; wave w owns 16 d_v columns of the fp32 state S^T (d_k x 16) in MFMA
// accumulators for the whole sequence.  Every state-dependent product (X1, Y,
// U, O, the state update) uses the previous result's accumulator tiles
// directly as the B operand of the next MFMA: a 16x16 accumulator holds rows
// 4g+i (g = lane/16) of column lane%16, which is a valid B fragment once the
// A operand reads its k index in the same order (k = 4g+i, then 16+4g+i).
// So the serial chain never leaves registers; shared per-chunk operands (K,
// Q, K^T, Tb, P) sit in LDS.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kCols = 64;  // d_v columns per workgroup (4 waves x 16)

// ------------------------------------------------------------------ MFMA
// A 32-deep k-step: lane l supplies 8 k values for row/column l%16, in the
// order k = 4g + j (j < 4) then 16 + 4g + (j - 4), g = l / 16.
template <typename T> struct Mma;

template <> struct Mma<__bf16> {
  using frag = bf16x8;
  static __device__ __forceinline__ frag zero() { return frag{}; }
  // from LDS row `row` (k contiguous): elements kb+4g..+3 and kb+16+4g..+3
  static __device__ __forceinline__ frag lds(const __bf16* row, int g, bool half) {
    const uint2 lo = *reinterpret_cast<const uint2*>(row + 4 * g);
    uint2 hi = make_uint2(0u, 0u);
    if (!half) hi = *reinterpret_cast<const uint2*>(row + 16 + 4 * g);
    return __builtin_bit_cast(frag, make_uint4(lo.x, lo.y, hi.x, hi.y));
  }
  // from two accumulator tiles (rows 4g+i of tile a, then of tile b)
  static __device__ __forceinline__ frag acc(const f32x4& a, const f32x4& b) {
    return __builtin_bit_cast(frag, make_uint4(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]),
                                               pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3])));
  }
  static __device__ __forceinline__ void mma(f32x4& c, const frag& a, const frag& b, bool half) {
    (void)half;
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mma<float> {
  struct frag { float v[8]; };
  static __device__ __forceinline__ frag zero() { frag f; for (int j = 0; j < 8; ++j) f.v[j] = 0.f; return f; }
  static __device__ __forceinline__ frag lds(const float* row, int g, bool half) {
    frag f;
    const float4 lo = *reinterpret_cast<const float4*>(row + 4 * g);
    float4 hi = make_float4(0.f, 0.f, 0.f, 0.f);
    if (!half) hi = *reinterpret_cast<const float4*>(row + 16 + 4 * g);
    f.v[0] = lo.x; f.v[1] = lo.y; f.v[2] = lo.z; f.v[3] = lo.w;
    f.v[4] = hi.x; f.v[5] = hi.y; f.v[6] = hi.z; f.v[7] = hi.w;
    return f;
  }
  static __device__ __forceinline__ frag acc(const f32x4& a, const f32x4& b) {
    frag f;
    for (int j = 0; j < 4; ++j) { f.v[j] = a[j]; f.v[4 + j] = b[j]; }
    return f;
  }
  // eight 16x16x4 fp32 MFMAs: MFMA j sums k = {4g + j} (j < 4) or {16 + 4g + j - 4}
  static __device__ __forceinline__ void mma(f32x4& c, const frag& a, const frag& b, bool half) {
#pragma unroll
    for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], c, 0, 0, 0);
    if (!half) {
#pragma unroll
      for (int j = 4; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], c, 0, 0, 0);
    }
  }
};

// ------------------------------------------------------------ LDS layout
template <typename T, int D, int C>
struct Layout {
  static constexpr int NT = C / 16;            // 16-token tiles per chunk
  static constexpr int DT = D / 16;            // 16-row tiles of d_k
  static constexpr int PADE = 32 / sizeof(T);  // 32 bytes of padding per row
  static constexpr int LDK = D + PADE;         // pitch of K, Q rows (token-major)
  static constexpr int LDC = C + PADE;         // pitch of K^T, Tb, P rows
  static constexpr int LDF = C + 4;            // pitch of fp32 A / T work arrays
  // byte offsets
  static constexpr int oK = 0;
  static constexpr int oQ = oK + C * LDK * (int)sizeof(T);
  static constexpr int oKT = oQ + C * LDK * (int)sizeof(T);
  static constexpr int oTb = oKT + D * LDC * (int)sizeof(T);
  static constexpr int oP = oTb + C * LDC * (int)sizeof(T);
  static constexpr int oA = oP + C * LDC * (int)sizeof(T);
  static constexpr int oTf = oA + C * LDF * 4;
  static constexpr int oZ = oTf + C * LDF * 4;          // 16 x C fp32 scratch
  static constexpr int oVec = oZ + 16 * LDF * 4;        // per-token fp32 vectors
  static constexpr int NVEC = 8;                        // g, beta, G, gamma*rk, scale*gamma*rq, e*rk, rk, rq
  static constexpr int bytes = oVec + NVEC * C * 4 + 16;
};

__device__ __forceinline__ float fexp(float x) { return __expf(x); }

// Accumulator tile 2s+1 of a chunk, or zeros when the chunk has an odd
// number of 16-token tiles (the second half of the last k-step is empty).
template <int NT>
__device__ __forceinline__ f32x4 tile_hi(const f32x4 (&t)[NT], int s) {
  const int i = 2 * s + 1;
  return i < NT ? t[i < NT ? i : 0] : f32x4{0.f, 0.f, 0.f, 0.f};
}

template <typename T, int D, int C>
__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillParams p) {
  using L = Layout<T, D, C>;
  using M = Mma<T>;
  constexpr int NT = L::NT, DT = L::DT;
  extern __shared__ __align__(16) unsigned char smem[];
  T* K_s = reinterpret_cast<T*>(smem + L::oK);
  T* Q_s = reinterpret_cast<T*>(smem + L::oQ);
  T* KT_s = reinterpret_cast<T*>(smem + L::oKT);
  T* Tb_s = reinterpret_cast<T*>(smem + L::oTb);
  T* P_s = reinterpret_cast<T*>(smem + L::oP);
  float* A_s = reinterpret_cast<float*>(smem + L::oA);
  float* T_s = reinterpret_cast<float*>(smem + L::oTf);
  float* Z_s = reinterpret_cast<float*>(smem + L::oZ);
  float* vec = reinterpret_cast<float*>(smem + L::oVec);
  float* g_s = vec;            // g
  float* b_s = vec + C;        // beta
  float* G_s = vec + 2 * C;    // cumulative g
  float* grk_s = vec + 3 * C;  // gamma_r rk_r
  float* grq_s = vec + 4 * C;  // scale gamma_r rq_r
  float* erk_s = vec + 5 * C;  // e_r rk_r
  float* rk_s = vec + 6 * C;
  float* rq_s = vec + 7 * C;
  float* misc = vec + 8 * C;   // [0] = gamma_{L-1}

  const int nblk = D / kCols > 0 ? D / kCols : 1;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = lane >> 4, l16 = lane & 15;
  const int blk = blockIdx.x % nblk;
  const int h = (blockIdx.x / nblk) % p.h_v;
  const int n = blockIdx.x / (nblk * p.h_v);
  const int hq = h / (p.h_v / p.h_qk);
  const int col = blk * kCols + wave * 16 + l16;  // this lane's d_v column
  const bool col_ok = col < D;                    // D = 64 uses one block of 64

  const int64_t seq_start = p.cu_seqlens ? p.cu_seqlens[n] : 0;
  const int64_t seq_end = p.cu_seqlens ? p.cu_seqlens[n + 1] : p.total_tokens;

  const T* qg = reinterpret_cast<const T*>(p.q) + (int64_t)hq * D;
  const T* kg = reinterpret_cast<const T*>(p.k) + (int64_t)hq * D;
  const T* vg = reinterpret_cast<const T*>(p.v) + (int64_t)h * D;
  T* og = reinterpret_cast<T*>(p.o) + (int64_t)h * D;
  const int64_t o_stride = (int64_t)p.h_v * D;

  // ---- state S^T (d_k x 16 columns of this wave) in DT accumulator tiles
  f32x4 st[DT];
  const size_t sbase = ((size_t)n * p.h_v + h) * D * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    st[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (p.initial_state && col_ok) {
      const float4 v4 = *reinterpret_cast<const float4*>(p.initial_state + sbase + (size_t)col * D + dt * 16 + 4 * g4);
      st[dt] = f32x4{v4.x, v4.y, v4.z, v4.w};
    }
  }

  for (int64_t t0 = seq_start; t0 < seq_end; t0 += C) {
    const int Lc = (int)min((int64_t)C, seq_end - t0);

    // ================= chunk prep (state independent) =================
    // K, Q rows -> LDS (token-major) and K^T (d_k-major); rows >= Lc are zero
    for (int e = tid; e < C * (D / 8); e += kThreads) {
      const int r = e / (D / 8);
      const int d0 = (e % (D / 8)) * 8;
      float kv[8], qv[8];
      if (r < Lc) {
        load8(kg + (t0 + r) * p.k_stride + d0, kv);
        load8(qg + (t0 + r) * p.q_stride + d0, qv);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) { kv[j] = 0.f; qv[j] = 0.f; }
      }
      store8(K_s + r * L::LDK + d0, kv);
      store8(Q_s + r * L::LDK + d0, qv);
#pragma unroll
      for (int j = 0; j < 8; ++j) KT_s[(d0 + j) * L::LDC + r] = from_f32<T>(kv[j]);
    }
    if (tid < C) {
      const bool ok = tid < Lc;
      g_s[tid] = ok ? p.g[(t0 + tid) * p.h_v + h] : 0.f;
      b_s[tid] = ok ? p.beta[(t0 + tid) * p.h_v + h] : 0.f;
    }
    __syncthreads();

    // row norms (4 lanes per row) and the cumulative log-decay (wave 0)
    for (int r = tid >> 2; r < C; r += kThreads / 4) {
      const int part = tid & 3;
      float sk = 0.f, sq = 0.f;
      for (int d = part; d < D; d += 4) {
        const float a = to_f32(K_s[r * L::LDK + d]);
        const float b = to_f32(Q_s[r * L::LDK + d]);
        sk += a * a; sq += b * b;
      }
      sk += dpp_f32<DPP_QUAD_1032>(sk); sk += dpp_f32<DPP_QUAD_2301>(sk);
      sq += dpp_f32<DPP_QUAD_1032>(sq); sq += dpp_f32<DPP_QUAD_2301>(sq);
      if (part == 0) {
        rk_s[r] = p.l2norm ? 1.0f / sqrtf(sk + 1e-6f) : 1.0f;
        rq_s[r] = p.l2norm ? 1.0f / sqrtf(sq + 1e-6f) : 1.0f;
      }
    }
    if (wave == 0) {
      float G = lane < C ? g_s[lane] : 0.f;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float o = __shfl_up(G, off, 64);
        if (lane >= off) G += o;
      }
      if (lane < C) G_s[lane] = G;
    }
    __syncthreads();
    if (tid < C) {
      const float Gl = G_s[Lc - 1];
      const float G = G_s[tid];
      grk_s[tid] = fexp(G) * rk_s[tid];
      grq_s[tid] = p.scale * fexp(G) * rq_s[tid];
      erk_s[tid] = fexp(Gl - G) * rk_s[tid];
      if (tid == 0) misc[0] = fexp(Gl);
    }

    // Gram tiles: KK^T -> A (strict lower, fp32), QK^T -> P (lower incl. diagonal)
    constexpr int NLT = NT * (NT + 1) / 2;
    for (int job = wave; job < 2 * NLT; job += 4) {
      const bool isP = job >= NLT;
      int tj = isP ? job - NLT : job;
      int mt = 0;
      while (tj > mt) { tj -= mt + 1; ++mt; }
      const int nt = tj;  // nt <= mt
      const T* Arow = (isP ? Q_s : K_s) + (mt * 16 + l16) * L::LDK;
      const T* Brow = K_s + (nt * 16 + l16) * L::LDK;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < D / 32; ++s)
        M::mma(acc, M::lds(Arow + 32 * s, g4, false), M::lds(Brow + 32 * s, g4, false), false);
      const int j = nt * 16 + l16;
      // G_s, b_s and the norms were published before the last barrier
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = mt * 16 + 4 * g4 + i;
        const float dec = (j <= r) ? fexp(G_s[r] - G_s[j]) : 0.f;
        if (!isP) {
          A_s[r * L::LDF + j] = (j < r) ? b_s[r] * dec * rk_s[r] * rk_s[j] * acc[i] : 0.f;
        } else {
          P_s[r * L::LDC + j] = from_f32<T>((j <= r) ? p.scale * dec * rq_s[r] * rk_s[j] * acc[i] : 0.f);
        }
      }
    }
    // upper tiles of P are zero
    for (int e = tid; e < C * C; e += kThreads) {
      const int r = e / C, j = e % C;
      if ((j >> 4) > (r >> 4)) P_s[r * L::LDC + j] = from_f32<T>(0.f);
    }
    __syncthreads();

    // T = (I + A)^-1: diagonal 16x16 blocks by forward substitution ...
    if (wave < NT && l16 == lane) {
      const int b = wave, c = lane;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float s = (r == c) ? 1.f : 0.f;
#pragma unroll
        for (int j = 0; j < r; ++j) s -= A_s[(16 * b + r) * L::LDF + 16 * b + j] * x[j];
        x[r] = s;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) T_s[(16 * b + r) * L::LDF + 16 * b + c] = x[r];
    }
    for (int e = tid; e < C * C; e += kThreads) {
      const int r = e / C, j = e % C;
      if ((j >> 4) > (r >> 4)) T_s[r * L::LDF + j] = 0.f;
    }
    __syncthreads();
    // ... then block rows: T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj
    for (int bi = 1; bi < NT; ++bi) {
      for (int e = tid; e < bi * 256; e += kThreads) {
        const int bj = e >> 8, rr = (e >> 4) & 15, cc = e & 15;
        float z = 0.f;
        for (int k = 16 * bj; k < 16 * bi; ++k)
          z += A_s[(16 * bi + rr) * L::LDF + k] * T_s[k * L::LDF + 16 * bj + cc];
        Z_s[rr * L::LDF + 16 * bj + cc] = z;
      }
      __syncthreads();
      for (int e = tid; e < bi * 256; e += kThreads) {
        const int bj = e >> 8, rr = (e >> 4) & 15, cc = e & 15;
        float t = 0.f;
#pragma unroll
        for (int m = 0; m < 16; ++m)
          t -= T_s[(16 * bi + rr) * L::LDF + 16 * bi + m] * Z_s[m * L::LDF + 16 * bj + cc];
        T_s[(16 * bi + rr) * L::LDF + 16 * bj + cc] = t;
      }
      __syncthreads();
    }
    // Tb = T diag(beta)
    for (int e = tid; e < C * C; e += kThreads) {
      const int r = e / C, j = e % C;
      Tb_s[r * L::LDC + j] = from_f32<T>(T_s[r * L::LDF + j] * b_s[j]);
    }
    __syncthreads();

    // ================= state-dependent chain (per wave) =================
    f32x4 x1[NT], yq[NT];
#pragma unroll
    for (int mt = 0; mt < NT; ++mt) { x1[mt] = f32x4{0.f, 0.f, 0.f, 0.f}; yq[mt] = x1[mt]; }
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      const typename M::frag bs = M::acc(st[2 * s], st[2 * s + 1]);
#pragma unroll
      for (int mt = 0; mt < NT; ++mt) {
        const int row = (mt * 16 + l16) * L::LDK + 32 * s;
        M::mma(x1[mt], M::lds(K_s + row, g4, false), bs, false);
        M::mma(yq[mt], M::lds(Q_s + row, g4, false), bs, false);
      }
    }
    // R = V - diag(gamma rk) X1   (in place in x1)
#pragma unroll
    for (int mt = 0; mt < NT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = mt * 16 + 4 * g4 + i;
        const float vv = (r < Lc && col_ok) ? to_f32(vg[(t0 + r) * p.v_stride + col]) : 0.f;
        x1[mt][i] = vv - grk_s[r] * x1[mt][i];
      }
    // U = Tb R
    f32x4 u[NT];
#pragma unroll
    for (int mt = 0; mt < NT; ++mt) u[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < (NT + 1) / 2; ++s) {
      const bool half = 2 * s + 1 >= NT;
      const typename M::frag bs = M::acc(x1[2 * s], tile_hi<NT>(x1, s));
#pragma unroll
      for (int mt = 0; mt < NT; ++mt)
        M::mma(u[mt], M::lds(Tb_s + (mt * 16 + l16) * L::LDC + 32 * s, g4, half), bs, half);
    }
    // O = diag(scale gamma rq) Y + P U
#pragma unroll
    for (int mt = 0; mt < NT; ++mt) x1[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < (NT + 1) / 2; ++s) {
      const bool half = 2 * s + 1 >= NT;
      const typename M::frag bs = M::acc(u[2 * s], tile_hi<NT>(u, s));
#pragma unroll
      for (int mt = 0; mt < NT; ++mt)
        M::mma(x1[mt], M::lds(P_s + (mt * 16 + l16) * L::LDC + 32 * s, g4, half), bs, half);
    }
#pragma unroll
    for (int mt = 0; mt < NT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = mt * 16 + 4 * g4 + i;
        if (r < Lc && col_ok)
          og[(t0 + r) * o_stride + col] = from_f32<T>(x1[mt][i] + grq_s[r] * yq[mt][i]);
      }
    // S^T <- gamma_last S^T + K^T diag(e rk) U
    const float gl = misc[0];
#pragma unroll
    for (int mt = 0; mt < NT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) u[mt][i] *= erk_s[mt * 16 + 4 * g4 + i];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) st[dt] *= gl;
#pragma unroll
    for (int s = 0; s < (NT + 1) / 2; ++s) {
      const bool half = 2 * s + 1 >= NT;
      const typename M::frag bs = M::acc(u[2 * s], tile_hi<NT>(u, s));
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        M::mma(st[dt], M::lds(KT_s + (dt * 16 + l16) * L::LDC + 32 * s, g4, half), bs, half);
    }
    __syncthreads();  // LDS is rewritten by the next chunk
  }

  if (p.final_state && col_ok) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<float4*>(p.final_state + sbase + (size_t)col * D + dt * 16 + 4 * g4) =
          make_float4(st[dt][0], st[dt][1], st[dt][2], st[dt][3]);
  }
}

template <typename T, int D, int C>
hipError_t launch_t(const PrefillParams& p, hipStream_t stream) {
  using L = Layout<T, D, C>;
  if constexpr (L::bytes > 160 * 1024) {
    return hipErrorInvalidConfiguration;  // rejected by prefill_supported() first
  } else {
    auto kern = prefill_kernel<T, D, C>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, L::bytes);
    if (e != hipSuccess) return e;
    const int nblk = D / kCols > 0 ? D / kCols : 1;
    const unsigned blocks = (unsigned)((int64_t)p.n_seqs * p.h_v * nblk);
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(kThreads), L::bytes, stream, p);
    return hipGetLastError();
  }
}

template <typename T, int D>
constexpr int lds_bytes(int chunk) {
  return chunk == 16 ? Layout<T, D, 16>::bytes : chunk == 32 ? Layout<T, D, 32>::bytes
                                                             : Layout<T, D, 64>::bytes;
}

template <typename T, int D>
hipError_t launch_c(const PrefillParams& p, hipStream_t stream) {
  switch (p.chunk) {
    case 16: return launch_t<T, D, 16>(p, stream);
    case 32: return launch_t<T, D, 32>(p, stream);
    default: return launch_t<T, D, 64>(p, stream);
  }
}

}  // namespace

size_t prefill_workspace_bytes(int64_t, int, int, int, int, int) { return 0; }

bool prefill_supported(int io_dtype, int d, int chunk) {
  const int b = io_dtype == 1 ? (d == 128 ? lds_bytes<__bf16, 128>(chunk) : lds_bytes<__bf16, 64>(chunk))
                              : (d == 128 ? lds_bytes<float, 128>(chunk) : lds_bytes<float, 64>(chunk));
  return b <= 160 * 1024;
}

hipError_t launch_prefill(const PrefillParams& p, int io_dtype, int d, hipStream_t stream) {
  if (io_dtype == 1) return d == 128 ? launch_c<__bf16, 128>(p, stream) : launch_c<__bf16, 64>(p, stream);
  return d == 128 ? launch_c<float, 128>(p, stream) : launch_c<float, 64>(p, stream);
}

}  // namespace gdn
