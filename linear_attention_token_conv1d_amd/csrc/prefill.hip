// gdn_prefill: chunked gated delta rule on gfx950.
//
// Math (per sequence and V head; within a chunk of L <= C tokens, G_r is the
// inclusive cumulative sum of g, gamma_r = e^{G_r}, e_r = e^{G_{L-1} - G_r},
// and k^_r = rk_r k_r, q^_r = rq_r q_r are the L2-normalised rows):
//   A_rj  = beta_r e^{G_r - G_j} (k^_r . k^_j)            j <  r   (strict lower)
//   T     = (I + A)^-1,   Tb = T diag(beta)
//   P_rj  = scale e^{G_r - G_j} (q^_r . k^_j)              j <= r
//   X1    = K S^T,  Y = Q S^T                   (raw K, Q rows)
//   R     = V - diag(gamma rk) X1
//   U     = Tb R                                (the chunk's delta writes)
//   O     = diag(scale gamma rq) Y + P U
//   S^T  <- gamma_{L-1} S^T + K^T diag(e rk) U
// This is the recurrence S_t = a_t S_{t-1}(I - b_t k_t k_t^T) + b_t v_t k_t^T,
// o_t = scale S_t q_t ("Inside Qwen3.5", sections 4-5) unrolled over one
// chunk; only e^{x} with x <= 0 is ever formed.
//
// Launches on the caller's stream:
//  plan  with cu_seqlens only, one workgroup: chunk offsets of every packed
//        sequence and the scan order (longest sequence first), in the
//        workspace (one sequence needs none: PlanView).
//  prep  one workgroup per (chunk, group of V heads sharing a QK head), all
//        chunks in parallel: row norms, the two Gram matrices (MFMA), the
//        decay masks, the UT solve T = (I + A)^-1 (forward substitution on
//        the diagonal blocks, fp32 MFMA below them) and the chunk operands
//        Tb, P and the per-token scalars, written to workspace.
//  scan  bf16: scan2_kernel, one workgroup per (sequence, V head, block of
//        32 or 64 d_v columns) walking its chunks in order.  Chain waves own
//        16 columns of the fp32 state S^T each in MFMA accumulators for the
//        whole sequence; every state-dependent product uses the previous
//        result's accumulator tiles directly as the B operand of the next
//        MFMA (a 16x16 accumulator holds rows 4g+i, g = lane/16, of column
//        lane%16: a valid B fragment once the A operand reads its k index in
//        the same order), so the serial chain never leaves registers.  Output
//        waves form O^T from the published state and U; mover waves (else
//        the output waves) bring the next chunk into the second LDS buffer
//        by direct-to-LDS loads.  fp32: scan_kernel, the same math in four
//        waves.
//  join  only after a split scan of one long sequence (see split_plan):
//        adds S_m w_t to the second segment's outputs and forms the final
//        state.
#include <cstdlib>
#include <mutex>
#include <type_traits>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kPrepThreads = 256;

// ------------------------------------------------------------------ MFMA
// A 32-deep k-step: lane l supplies 8 k values for row/column l%16, in the
// order k = 4g + j (j < 4) then 16 + 4g + (j - 4), g = l / 16.
template <typename T> struct Mma;

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4;

template <> struct Mma<__bf16> {
  using frag = bf16x8;
  // from LDS row `row` (k contiguous): elements 4g..4g+3 and 16+4g..16+4g+3
  static __device__ __forceinline__ frag lds(const __bf16* row, int g, bool half) {
    const uint2 lo = *reinterpret_cast<const uint2*>(row + 4 * g);
    uint2 hi = make_uint2(0u, 0u);
    if (!half) hi = *reinterpret_cast<const uint2*>(row + 16 + 4 * g);
    return __builtin_bit_cast(frag, make_uint4(lo.x, lo.y, hi.x, hi.y));
  }
  // K^T fragment (m = d_k column dcol0 + lane%16, k = token) from the
  // row-major tile K[token][d_k] at tokens tok0 + 4g + {0..3} and +16.  In
  // each 16-lane group, lane j reads 4 consecutive d_k of token 4g + j/4; the
  // transpose read hands lane i element i%4 of the rows read by lanes
  // i/4 + 4e (e = 0..3), i.e. K[tok0 + 4g + e][dcol0 + i].
  static __device__ __forceinline__ frag lds_tr(const __bf16* K, int ld, int tok0, int dcol0, int l16,
                                                int g, bool half) {
    const __bf16* p = K + (tok0 + 4 * g + (l16 >> 2)) * ld + dcol0 + 4 * (l16 & 3);
    const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_short4*)(__attribute__((address_space(3))) __bf16*)(p));
    short4_t hi = {0, 0, 0, 0};
    if (!half)
      hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_short4*)(__attribute__((address_space(3))) __bf16*)(p + 16 * ld));
    const uint2 a = __builtin_bit_cast(uint2, lo), b = __builtin_bit_cast(uint2, hi);
    return __builtin_bit_cast(frag, make_uint4(a.x, a.y, b.x, b.y));
  }
  // from two accumulator tiles (rows 4g+i of tile a, then of tile b)
  static __device__ __forceinline__ frag acc(const f32x4& a, const f32x4& b) {
    return __builtin_bit_cast(frag, make_uint4(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]),
                                               pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3])));
  }
  static __device__ __forceinline__ void mma(f32x4& c, const frag& a, const frag& b, bool) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mma<float> {
  struct frag { float v[8]; };
  static __device__ __forceinline__ frag lds(const float* row, int g, bool half) {
    frag f;
    const float4 lo = *reinterpret_cast<const float4*>(row + 4 * g);
    float4 hi = make_float4(0.f, 0.f, 0.f, 0.f);
    if (!half) hi = *reinterpret_cast<const float4*>(row + 16 + 4 * g);
    f.v[0] = lo.x; f.v[1] = lo.y; f.v[2] = lo.z; f.v[3] = lo.w;
    f.v[4] = hi.x; f.v[5] = hi.y; f.v[6] = hi.z; f.v[7] = hi.w;
    return f;
  }
  static __device__ __forceinline__ frag lds_tr(const float* K, int ld, int tok0, int dcol0, int l16,
                                                int g, bool half) {
    frag f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f.v[e] = K[(tok0 + 4 * g + e) * ld + dcol0 + l16];
      f.v[4 + e] = half ? 0.f : K[(tok0 + 16 + 4 * g + e) * ld + dcol0 + l16];
    }
    return f;
  }
  static __device__ __forceinline__ frag acc(const f32x4& a, const f32x4& b) {
    frag f;
#pragma unroll
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

// 8 consecutive elements as raw bits (16 B of bf16, 32 B of fp32)
template <typename T> struct Raw8;
template <> struct Raw8<__bf16> {
  uint4 a;
  static __device__ __forceinline__ Raw8 load(const __bf16* p) { return {*reinterpret_cast<const uint4*>(p)}; }
  static __device__ __forceinline__ Raw8 zero() { return {make_uint4(0u, 0u, 0u, 0u)}; }
  __device__ __forceinline__ void store(__bf16* p) const { *reinterpret_cast<uint4*>(p) = a; }
};
template <> struct Raw8<float> {
  uint4 a, b;
  static __device__ __forceinline__ Raw8 load(const float* p) {
    return {reinterpret_cast<const uint4*>(p)[0], reinterpret_cast<const uint4*>(p)[1]};
  }
  static __device__ __forceinline__ Raw8 zero() { return {make_uint4(0u, 0u, 0u, 0u), make_uint4(0u, 0u, 0u, 0u)}; }
  __device__ __forceinline__ void store(float* p) const {
    reinterpret_cast<uint4*>(p)[0] = a;
    reinterpret_cast<uint4*>(p)[1] = b;
  }
};

__device__ __forceinline__ float fexp(float x) { return __expf(x); }

// Four consecutive elements of a caller's state tensor (fp32, or bf16 when
// the call stores its states as bf16), at element offset i (a multiple of 4).
__device__ __forceinline__ f32x4 load_state4(const void* base, size_t i, bool bf16) {
  if (bf16) {
    const uint2 w = *reinterpret_cast<const uint2*>(reinterpret_cast<const __bf16*>(base) + i);
    return f32x4{bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y)};
  }
  const float4 v = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + i);
  return f32x4{v.x, v.y, v.z, v.w};
}
__device__ __forceinline__ void store_state4(void* base, size_t i, const f32x4& v, bool bf16) {
  if (bf16)
    *reinterpret_cast<uint2*>(reinterpret_cast<__bf16*>(base) + i) =
        make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
  else
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(base) + i) = make_float4(v[0], v[1], v[2], v[3]);
}

// Accumulator tile 2s+1 of a chunk, or zeros when the chunk has an odd
// number of 16-token tiles (the second half of the last k-step is empty).
template <int NT>
__device__ __forceinline__ f32x4 tile_hi(const f32x4 (&t)[NT], int s) {
  const int i = 2 * s + 1;
  return i < NT ? t[i < NT ? i : 0] : f32x4{0.f, 0.f, 0.f, 0.f};
}

// Y^T W + acc for 16x16 fp32 tiles held in the accumulator layout (lane
// (g, c) holds rows 4g..4g+3 of column c): MFMA s sums over k = 4g + s, its
// A operand being register s of Y's tile (Y[4g+s][c] = Y^T[c][4g+s]) and its
// B operand register s of W's tile.
__device__ __forceinline__ f32x4 mfma_tn(const f32x4& y, const f32x4& w, f32x4 acc) {
#pragma unroll
  for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(y[s], w[s], acc, 0, 0, 0);
  return acc;
}

// ------------------------------------------------------------- workspace
// [chunk offsets: n_seqs+1 int32, scan order: n_seqs int32, padded to 256 B]
// [per (chunk, V head) record: Tb [C][C] T | P [C][C] T | vec [4][C] fp32]
//  vec rows: gamma*rk, scale*gamma*rq, e*rk, gamma_last (broadcast)
template <typename T, int C>
struct Rec {
  static constexpr size_t mat = (size_t)C * C * sizeof(T);
  static constexpr size_t bytes = 2 * mat + 16 * (size_t)C;
};

// [chunk offsets: n_seqs+1 int32 | scan order: n_seqs int32 | rows of the
//  emitted chunk-boundary states: n_seqs+1 int32], padded to 256 B
__host__ __device__ constexpr size_t off_bytes(int n_seqs) { return (((size_t)n_seqs * 3 + 2) * 4 + 255) / 256 * 256; }

__host__ __device__ inline int64_t max_chunks(int64_t T, int n_seqs, int C) { return T / C + n_seqs; }

// Sequence split of the bf16 scan.  When one sequence's heads leave most CUs
// idle, its chunks [0, m) are scanned from the initial state (ending in S_m)
// while chunks [m, nch) are scanned twice at the same time: from a zero state
// (outputs o0, final state S0) and as the transition Phi of that segment
// (basis initial state, zero values: outputs w_t = scale Phi_{m,t} q^_t, final
// state Phi).  Every state update is linear in the state, so on the second
// segment o_t = o0_t + S_m w_t and the final state is S_m Phi + S0; a join
// launch forms both.  Workspace after the records, 256-byte aligned:
// [S_m | S0 | Phi: h_v d d fp32 each][w: tokens of the second segment x h_v x d, bf16]
constexpr int kSplitMinChunks = 32;  // shorter sequences keep one pass
constexpr int kScanCUs = 256;
struct SplitPlan {
  bool on;
  int cols;          // columns per scan workgroup (32 or 64)
  int m;             // chunks in the first segment
  int64_t t_b;       // first token of the second segment
  size_t o_state, o_w, o_smb, bytes;  // workspace offsets (after the records) and total
};
__host__ __device__ inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }
inline SplitPlan split_plan(int io_dtype, int64_t T, int n_seqs, int h_v, int d, int C, int emit_every,
                            size_t base) {
  SplitPlan s{false, 0, 0, 0, 0, 0, 0, base};
  const int64_t nch = (T + C - 1) / C;
  // chunk-boundary states are not formed on the second segment: no split then
  if (io_dtype != 1 || n_seqs != 1 || emit_every > 0 || nch < kSplitMinChunks) return s;
  // Workgroups of one role (first segment, second from zero, transition):
  // gn with 32 columns, gw with 64.  The first segment's go first in the
  // grid.  If all three roles fit on the CUs, the halves are even.  If only
  // the first segment and part of the second fit, the rest of the second
  // segment starts as its first workgroups finish: the second segment then
  // runs in two waves and gets a third of the chunks.
  const int gn = h_v * (d / 32), gw = h_v * (d / 64);
  if (3 * gn <= kScanCUs) {
    s.cols = 32;
    s.m = (int)(nch / 2);
  } else if (2 * gn <= kScanCUs) {
    s.cols = 32;
    s.m = (int)((2 * nch + 1) / 3);
  } else if (3 * gw <= kScanCUs) {
    s.cols = 64;
    s.m = (int)(nch / 2);
  } else {
    return s;
  }
  s.on = true;
  s.t_b = (int64_t)s.m * C;
  s.o_state = align256(base);
  s.o_w = s.o_state + 3 * (size_t)h_v * d * d * 4;
  s.o_smb = align256(s.o_w + (size_t)(T - s.t_b) * h_v * d * 2);
  s.bytes = align256(s.o_smb + (size_t)h_v * d * d * 2);
  return s;
}
// What a split scan's workgroups find: role 0 = first segment, 1 = second
// segment from zero, 2 = the transition of the second segment.
struct ScanSplit {
  int on, m;
  float* s_mid;  // [h_v][d][d] state after chunk m
  float* s_zero; // [h_v][d][d] second segment's final state from zero
  float* phi;    // [h_v][d][d] transition of the second segment (row i = basis row i)
  __bf16* w;     // [tokens after t_b][h_v][d]
  __bf16* s_mid_bf;  // [h_v][d][d] S_m rounded to bf16 (the join's MFMA operand)
};

// 256 zero bytes: the V rows of the transition role of a split scan
__device__ __align__(256) unsigned char g_zero_line[256] = {};

// ------------------------------------------------------------------ plan
// One workgroup: chunk offsets of every packed sequence (exclusive prefix sum
// of ceil(len / C)), then the scan order: sequences by chunk count, longest
// first (ties by index), so that the longest serial chains start first.
constexpr int kPlanSortMax = 2048;  // longer batches keep their own order

__global__ __launch_bounds__(256) void plan_kernel(const int32_t* cu, int n_seqs, int64_t total, int C,
                                                   int emit_every, int32_t* chunk_off) {
  __shared__ int32_t part[256];
  __shared__ int32_t carry;
  __shared__ int32_t cnt_s[kPlanSortMax];
  const int tid = threadIdx.x;
  // out[0] = 0, out[i + 1] = sum of count(m) over m <= i
  auto prefix = [&](auto count, int32_t* out) {
    if (tid == 0) { carry = 0; out[0] = 0; }
    __syncthreads();
    for (int base = 0; base < n_seqs; base += 256) {
      const int i = base + tid;
      part[tid] = i < n_seqs ? count(i) : 0;
      __syncthreads();
      for (int o = 1; o < 256; o <<= 1) {
        const int v = tid >= o ? part[tid - o] : 0;
        __syncthreads();
        part[tid] += v;
        __syncthreads();
      }
      if (i < n_seqs) out[i + 1] = carry + part[tid];
      __syncthreads();
      if (tid == 255) carry += part[255];
      __syncthreads();
    }
  };
  auto len = [&](int i) { return cu ? (int64_t)cu[i + 1] - cu[i] : total; };
  // chunks per sequence (kept for the scan order)
  prefix([&](int i) {
    const int cnt = (int)((len(i) + C - 1) / C);
    if (i < kPlanSortMax) cnt_s[i] = cnt;
    return cnt;
  }, chunk_off);
  // emitted chunk-boundary states per sequence: boundaries j K C < len
  if (emit_every > 0) {
    const int64_t every = (int64_t)emit_every * C;
    prefix([&](int i) { return (int)(len(i) > 0 ? (len(i) - 1) / every : 0); }, chunk_off + 2 * n_seqs + 1);
  }
  int32_t* order = chunk_off + n_seqs + 1;
  for (int i = tid; i < n_seqs; i += 256) {
    int rank = i;
    if (n_seqs <= kPlanSortMax) {
      const int ci = cnt_s[i];
      rank = 0;
      for (int j = 0; j < n_seqs; ++j) {
        const int cj = cnt_s[j];
        rank += (cj > ci) || (cj == ci && j < i);
      }
    }
    order[rank] = i;
  }
}

// The plan's arrays as the kernels read them.  A call with one sequence and
// no cu_seqlens launches no plan: each value follows from the token count.
struct PlanView {
  cint32* a;  // chunk offsets | scan order | emission rows, or null
  int n_seqs;
  int nch1;   // chunks of the one sequence when a is null
  __device__ __forceinline__ int off(int i) const { return a ? a[i] : i == 0 ? 0 : nch1; }
  __device__ __forceinline__ int order(int i) const { return a ? a[n_seqs + 1 + i] : 0; }
  __device__ __forceinline__ int erow(int n) const { return a ? a[2 * n_seqs + 1 + n] : 0; }
};
__device__ __forceinline__ PlanView plan_view(const PrefillParams& p, const unsigned char* ws, int C) {
  return PlanView{p.cu_seqlens ? as_const(reinterpret_cast<const int32_t*>(ws)) : nullptr, p.n_seqs,
                  (int)((p.total_tokens + C - 1) / C)};
}

// Workgroup -> (sequence, V head, column block) for the scans.  The unit of
// placement is a QK-head group: the grp = h_v / h_qk V heads (times NB column
// blocks) that read the same K, Q and chunk rows.  Consecutive groups go to
// consecutive XCDs (the hardware deals workgroups round-robin over the 8
// XCDs), so one group shares an L2 while long chains spread over all XCDs;
// groups are numbered in scan order (longest sequence first).
struct ScanSlot {
  int n, h, blk, role;
  bool valid;
};
__device__ __forceinline__ ScanSlot scan_slot(const PrefillParams& p, const PlanView& pv, int NB) {
  const int grp = p.h_v / p.h_qk, gs = grp * NB, ngroups = p.n_seqs * p.h_qk;
  const int x = blockIdx.x % 8, k = blockIdx.x / 8;
  const int gi = (k / gs) * 8 + x, j = k % gs;
  ScanSlot r{0, 0, 0, 0, gi < ngroups};
  if (r.valid) {
    r.n = pv.order(gi / p.h_qk);
    r.h = (gi % p.h_qk) * grp + j / NB;
    r.blk = j % NB;
  }
  return r;
}
// Split scan of one sequence: the h_v NB first-segment workgroups come first
// in the grid (they must all start at once), then per V head the NB
// second-segment and NB transition workgroups, which read the same chunks.
// With h_v a multiple of 8 the heads go to the XCDs in runs (blockIdx mod 8
// is the XCD), so the workgroups of a head share one L2.
__device__ __forceinline__ ScanSlot split_slot(const PrefillParams& p, int NB) {
  const int G = p.h_v * NB, b = blockIdx.x;
  const bool first = b < G;
  const int per = first ? NB : 2 * NB, bb = first ? b : b - G;
  int h, j;
  if (p.h_v % 8 == 0) {
    const int x = bb % 8, k = bb / 8;
    h = x * (p.h_v / 8) + k / per;
    j = k % per;
  } else {
    h = bb / per;
    j = bb % per;
  }
  return ScanSlot{0, h, j % NB, first ? 0 : 1 + j / NB, h < p.h_v};
}
inline unsigned scan_grid(int n_seqs, int h_qk, int h_v, int NB) {
  const int ngroups = n_seqs * h_qk;
  return (unsigned)(8 * ((ngroups + 7) / 8) * (h_v / h_qk) * NB);
}

// ---------------------------------------------------- LDS tile helpers
// Row order inside a pair of 16-row MFMA tiles.  Row m of tile 2s+b stands
// for index 32s + 8(m/4) + 4b + m%4 (tokens of a chunk, or d_k of the state).
// An accumulator tile holds rows 4g+i (g = lane/16) of column lane%16; with
// this order the two tiles 2s, 2s+1 give lane group g the 8 consecutive
// indices 32s + 8g .. 32s + 8g + 7, so the B fragment built from them pairs
// with an A fragment that is one contiguous 16-byte read.  A chunk of 16
// tokens (a single tile) keeps the plain order and half-empty k-steps.
template <int NT>
__device__ __forceinline__ int pidx(int t, int m) {
  if constexpr (NT == 1) return m;
  else return 32 * (t >> 1) + 8 * (m >> 2) + 4 * (t & 1) + (m & 3);
}

// Swizzled LDS tiles.  A tile holds rows of RB bytes (RB/16 sixteen-byte
// chunks); chunk j of row r sits at slot j ^ f(r).  The two row functions
// below keep the 16-byte fragment reads (16 rows of one tile pair, one chunk)
// and the per-column V reads of a wave on distinct banks.  The layout is
// dense, so a wave's direct-to-LDS load (64 lanes x 16 B into 1 KiB of
// consecutive LDS) fills it without a register round trip.
// Row functions of the swizzles below (slot of chunk j of row r = j ^ f(r)).
struct RowK {  // token-major K/Q tiles of 16+ chunks: fragment rows in pidx order, transpose reads
  static __device__ __forceinline__ int f(int r) { return (2 * ((r & 3) | (((r >> 3) & 1) << 2))) | ((r >> 4) & 1); }
};
struct RowT {  // narrower tiles (Tb, P; K/Q when d_k = 64)
  static __device__ __forceinline__ int f(int r) { return ((r >> 1) & 1) | (((r >> 3) & 3) << 1); }
};
template <int NT, int CPR>
struct RowV {  // V tile read by the transposing loads: the rows a 32-lane pass reads on distinct banks
  static __device__ __forceinline__ int f(int r) {
    if constexpr (CPR >= 8) {
      if constexpr (NT == 1) return (((r >> 1) & 1) | (((r >> 2) & 1) << 1)) << 1;
      else return (((r >> 1) & 1) | (((r >> 3) & 1) << 1)) << 1;
    } else {
      if constexpr (NT == 1) return ((r >> 2) & 1) << 1;
      else return ((r >> 3) & 1) << 1;
    }
  }
};
template <int RB>
struct RowSeq {  // 16 consecutive rows read at one chunk: spread over the 256-byte bank window
  static __device__ __forceinline__ int f(int r) { return r / (RB >= 256 ? 1 : 256 / RB); }
};

template <int RB, typename F>
struct SwzT {
  static constexpr int CPR = RB / 16;
  static_assert(CPR >= 1 && (CPR & (CPR - 1)) == 0, "row of 2^k chunks");
  static constexpr int RBYTES = RB;
  static __device__ __forceinline__ int slot(int r, int j) { return (j ^ F::f(r)) & (CPR - 1); }
  // byte offset of byte b of row r
  static __device__ __forceinline__ int off(int r, int b) { return r * RB + (slot(r, b >> 4) << 4) + (b & 15); }
};
template <int RB>
using Swz = SwzT<RB, std::conditional_t<(RB / 16 >= 16), RowK, RowT>>;

// Direct-to-LDS copy of ROWS rows of RB bytes.  Global row r (clamped to
// rmax - 1) starts at gbase + r * gstride bytes.  Instruction k of wave w
// fills LDS chunks [(k * NWAVES + w) * 64, +64): lane l writes chunk q and
// fetches the global chunk whose swizzled slot is q.
template <typename S, int ROWS, int NWAVES>
__device__ __forceinline__ void dma_tile_s(unsigned char* lds, const unsigned char* gbase, int64_t gstride,
                                           int rmax, int wave, int lane) {
  constexpr int TOTAL = ROWS * S::CPR;
#pragma unroll
  for (int k = 0; k * NWAVES * 64 < TOTAL; ++k) {
    const int q0 = (k * NWAVES + wave) * 64;
    const int q = q0 + lane;
    if (q0 < TOTAL && q < TOTAL) {
      const int r = q / S::CPR;
      const int j = S::slot(r, q % S::CPR);  // slot(r, .) is an involution
      const unsigned char* src = gbase + (int64_t)min(r, rmax - 1) * gstride + j * 16;
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(lds + q0 * 16), 16, 0, 0);
    }
  }
}
template <int RB, int ROWS, int NWAVES>
__device__ __forceinline__ void dma_tile(unsigned char* lds, const unsigned char* gbase, int64_t gstride,
                                         int rmax, int wave, int lane) {
  dma_tile_s<Swz<RB>, ROWS, NWAVES>(lds, gbase, gstride, rmax, wave, lane);
}

// Plain direct-to-LDS copy of NB bytes (a multiple of 16).
template <int NB, int NWAVES>
__device__ __forceinline__ void dma_linear(unsigned char* lds, const unsigned char* g, int wave, int lane) {
  constexpr int TOTAL = NB / 16;
#pragma unroll
  for (int k = 0; k * NWAVES * 64 < TOTAL; ++k) {
    const int q0 = (k * NWAVES + wave) * 64;
    const int q = q0 + lane;
    if (q0 < TOTAL && q < TOTAL)
      __builtin_amdgcn_global_load_lds(g + q * 16, (__attribute__((address_space(3))) void*)(lds + q0 * 16), 16, 0, 0);
  }
}

// Precomputed form of dma_tile_s for full chunks: the per-lane source offset
// of each instruction (row r of the tile at r * gstride bytes, chunk slot
// from the swizzle) does not change from chunk to chunk, so it is computed
// once and a chunk costs one address add per instruction.  Offsets are 32-bit
// (the caller checks that ROWS * gstride fits).
template <typename S, int ROWS, int NWAVES>
struct DmaPlan {
  static constexpr int TOTAL = ROWS * S::CPR;
  static constexpr int NI = (TOTAL + NWAVES * 64 - 1) / (NWAVES * 64);
  uint32_t off[NI];
  __device__ __forceinline__ void init(uint32_t gstride, int wave, int lane) {
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      const int q = min((k * NWAVES + wave) * 64 + lane, TOTAL - 1);
      const int r = q / S::CPR;
      off[k] = (uint32_t)r * gstride + (uint32_t)S::slot(r, q % S::CPR) * 16u;
    }
  }
  // instruction k of this wave (no-op past the tile)
  __device__ __forceinline__ void issue_one(int k, unsigned char* lds, const unsigned char* gbase, int wave,
                                            int lane) const {
    const int q0 = (k * NWAVES + wave) * 64;
    if (q0 < TOTAL && q0 + lane < TOTAL)
      __builtin_amdgcn_global_load_lds(gbase + off[k], (__attribute__((address_space(3))) void*)(lds + q0 * 16), 16, 0, 0);
  }
  __device__ __forceinline__ void issue(unsigned char* lds, const unsigned char* gbase, int wave, int lane) const {
#pragma unroll
    for (int k = 0; k < NI; ++k) issue_one(k, lds, gbase, wave, lane);
  }
};

// A fragment: 8 consecutive elements k0..k0+7 of row `row` of a swizzled
// tile (4 elements and 4 zeros when `half`).
template <typename T, typename S>
__device__ __forceinline__ typename Mma<T>::frag frag_row_s(const unsigned char* tile, int row, int k0, bool half);
template <typename T, int RB>
__device__ __forceinline__ typename Mma<T>::frag frag_row(const unsigned char* tile, int row, int k0, bool half) {
  return frag_row_s<T, Swz<RB>>(tile, row, k0, half);
}
template <typename T, typename S>
__device__ __forceinline__ typename Mma<T>::frag frag_row_s(const unsigned char* tile, int row, int k0, bool half) {
  if constexpr (sizeof(T) == 2) {
    if (half) {
      const uint2 lo = *reinterpret_cast<const uint2*>(tile + S::off(row, k0 * 2));
      return __builtin_bit_cast(typename Mma<T>::frag, make_uint4(lo.x, lo.y, 0u, 0u));
    }
    return __builtin_bit_cast(typename Mma<T>::frag, *reinterpret_cast<const uint4*>(tile + S::off(row, k0 * 2)));
  } else {
    typename Mma<T>::frag f;
    const float4 lo = *reinterpret_cast<const float4*>(tile + S::off(row, k0 * 4));
    float4 hi = make_float4(0.f, 0.f, 0.f, 0.f);
    if (!half) hi = *reinterpret_cast<const float4*>(tile + S::off(row, k0 * 4 + 16));
    f.v[0] = lo.x; f.v[1] = lo.y; f.v[2] = lo.z; f.v[3] = lo.w;
    f.v[4] = hi.x; f.v[5] = hi.y; f.v[6] = hi.z; f.v[7] = hi.w;
    return f;
  }
}

// K^T fragment for the state update: rows m = d_k index dk(m) of state
// tile t, k = the 8 (or 4) tokens tok0 .. tok0+7 of lane group g, from the
// swizzled token-major K tile.  bf16: in each 16-lane group, lane j reads 4
// consecutive d_k (those of state rows 4(j%4)..4(j%4)+3) of token tok0 + j/4,
// and the transpose read hands lane i element i%4 of the rows read by lanes
// i/4 + 4e, i.e. K[tok0 + e][dk(i)]; the second read covers tok0 + 4..7.
template <typename T, int RB, int DTP>
__device__ __forceinline__ typename Mma<T>::frag frag_kt(const unsigned char* tile, int t, int tok0, int l16,
                                                         bool half) {
  using S = Swz<RB>;
  if constexpr (sizeof(T) == 2) {
    const int row = tok0 + (l16 >> 2);
    const int b = pidx<DTP>(t, 4 * (l16 & 3)) * 2;
    const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_short4*)(__attribute__((address_space(3))) unsigned char*)(tile + S::off(row, b)));
    short4_t hi = {0, 0, 0, 0};
    if (!half)
      hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_short4*)(__attribute__((address_space(3))) unsigned char*)(tile + S::off(row + 4, b)));
    const uint2 a = __builtin_bit_cast(uint2, lo), c = __builtin_bit_cast(uint2, hi);
    return __builtin_bit_cast(typename Mma<T>::frag, make_uint4(a.x, a.y, c.x, c.y));
  } else {
    typename Mma<T>::frag f;
    const int b = pidx<DTP>(t, l16) * 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f.v[e] = *reinterpret_cast<const float*>(tile + S::off(tok0 + e, b));
      f.v[4 + e] = half ? 0.f : *reinterpret_cast<const float*>(tile + S::off(tok0 + 4 + e, b));
    }
    return f;
  }
}

// ------------------------------------------------------------------ prep
// One workgroup per (chunk, V head).  The chunk's raw K and Q rows are loaded
// into registers (every load issued before any is used); their L2 norms are
// reduced there, then the rows go to swizzled LDS tiles for the Gram MFMAs.
// The Gram tiles are formed transposed (K Q^T, K K^T tile by tile), so a lane
// holds four consecutive columns of one row of P and of A: P goes straight
// to the workspace and A to the fp32 work array of the UT solve, which
// reuses the K/Q bytes.  Tb = T diag(beta) leaves in 16-byte row pieces.
template <typename T, int D, int C, int VPW>
struct PrepLayout {
  static constexpr int NT = C / 16;
  static constexpr int E = (int)sizeof(T);
  static constexpr int LDF = C + 4;
  // the K, Q tiles hold d_k in NH passes: two when they would otherwise be
  // the largest LDS user (one V head per workgroup)
  static constexpr int NH = 2 * C * D * E > VPW * C * LDF * 4 ? 2 : 1;
  static constexpr int DH = D / NH;
  static constexpr int RBH = DH * E;  // K, Q tile rows (swizzled)
  // phase 1 (shared by the V-head teams): K, Q tiles
  static constexpr int oK = 0;
  static constexpr int oQ = oK + C * RBH;
  static constexpr int kq_bytes = oQ + C * RBH;
  // phase 2 (same bytes): per team, the A/T work array
  static constexpr int oA = 0;
  static constexpr int team_bytes = oA + C * LDF * 4;
  static constexpr int work_bytes = VPW * team_bytes;
  // with several teams (one K, Q pass), the raw Gram tiles (fp32, 1 KiB
  // each) formed once for all teams and read by each team's masks
  static constexpr int NLT = NT * (NT + 1) / 2;
  static constexpr bool share = VPW > 1 && NH == 1;
  static constexpr int oStage = kq_bytes > work_bytes ? kq_bytes : work_bytes;
  // row scalars: rk, rq (shared), then g, beta, G per team
  static constexpr int oVec = oStage + (share ? 2 * NLT * 1024 : 0);
  static constexpr int bytes = oVec + (2 + 3 * VPW) * C * 4;
  // with split tiles, the waves per SIMD that LDS allows (at most 6) set the
  // register budget; otherwise the compiler's own choice stands
  static constexpr int wgs = 160 * 1024 / bytes;
  static constexpr int waves_per_eu = NH == 1 ? 1 : wgs * VPW > 6 ? 6 : wgs * VPW < 1 ? 1 : wgs * VPW;
};

// Largest n in [0, n_seqs) with off(n) <= c (the sequence owning chunk c).
__device__ __forceinline__ int owner(const PlanView& pv, int c) {
  int lo = 0, hi = pv.a ? pv.n_seqs - 1 : 0;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pv.off(mid) <= c) lo = mid; else hi = mid - 1;
  }
  return lo;
}

template <typename T, int D, int C, int VPW>
__global__ __launch_bounds__(kPrepThreads * VPW)
__attribute__((amdgpu_waves_per_eu(PrepLayout<T, D, C, VPW>::waves_per_eu))) void prep_kernel(PrefillParams p,
                                                                                             unsigned char* ws) {
  using L = PrepLayout<T, D, C, VPW>;
  using M = Mma<T>;
  using R8 = Raw8<T>;
  using SK = Swz<L::RBH>;
  constexpr int NT = L::NT;
  constexpr int NLT = NT * (NT + 1) / 2;       // lower-triangular 16x16 tiles
  constexpr int NJ = (2 * NLT + 3) / 4;        // masked tiles per team wave
  // Gram tiles: shared by all the workgroup's waves when teams share them
  constexpr int GW = L::share ? 4 * VPW : 4;
  constexpr int NJG = (2 * NLT + GW - 1) / GW;
  constexpr int RT = D / 8;                    // threads per row in the load layout
  constexpr int NTH = kPrepThreads * VPW;
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  // four waves (one team) per V head: the teams share the K, Q load, the
  // norms and the K, Q tiles, and run the per-V-head steps side by side
  const int team = tid / kPrepThreads, ttid = tid % kPrepThreads, wave = ttid >> 6;
  const int g4 = lane >> 4, l16 = lane & 15;
  unsigned char* K_s = smem + L::oK;
  unsigned char* Q_s = smem + L::oQ;
  float* A_s = reinterpret_cast<float*>(smem + team * L::team_bytes + L::oA);
  float* rk_s = reinterpret_cast<float*>(smem + L::oVec);
  float* rq_s = rk_s + C;
  float* g_s = rk_s + (2 + 3 * team) * C;
  float* b_s = g_s + C;
  float* G_s = g_s + 2 * C;

  const PlanView pv = plan_view(p, ws, C);
  cint32* cu = as_const(p.cu_seqlens);
  const int ci = blockIdx.x, h = blockIdx.y * VPW + team;
  if (ci >= pv.off(p.n_seqs)) return;
  const int hq = h / (p.h_v / p.h_qk);  // the same for every team (VPW divides h_v / h_qk)
  const int n = owner(pv, ci);
  const int64_t seq_start = cu ? cu[n] : 0;
  const int64_t seq_end = cu ? cu[n + 1] : p.total_tokens;
  const int64_t t0 = seq_start + (int64_t)(ci - pv.off(n)) * C;
  const int Lc = (int)min((int64_t)C, seq_end - t0);

  // K, Q rows of this chunk and QK head; g, beta of this V head.  Rows past
  // the chunk re-read its last row and are zeroed below.
  const T* kg = reinterpret_cast<const T*>(p.k) + (int64_t)hq * D;
  const T* qg = reinterpret_cast<const T*>(p.q) + (int64_t)hq * D;
  // piece (hf, e) of a pass: row e / RTH, d_k 8 (e % RTH) of part hf
  constexpr int RTH = RT / L::NH;                 // threads per row and part
  constexpr int NV = (C * RTH + NTH - 1) / NTH;   // pieces per thread and part
  R8 kv[L::NH][NV], qv[L::NH][NV];
#pragma unroll
  for (int hf = 0; hf < L::NH; ++hf)
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = min(tid + i * NTH, C * RTH - 1);
      const int r = min(e / RTH, Lc - 1), d0 = hf * L::DH + (e % RTH) * 8;
      kv[hf][i] = R8::load(kg + (t0 + r) * p.k_stride + d0);
      qv[hf][i] = R8::load(qg + (t0 + r) * p.q_stride + d0);
    }
  const int ti = min(ttid, Lc - 1);
  const float gv = p.g[(t0 + ti) * p.h_v + h];
  const float bv = p.beta[(t0 + ti) * p.h_v + h];

  // row norms: the RTH threads of a row are consecutive lanes; a thread
  // holds the same rows in every part
  float skr[NV], sqr[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) skr[i] = sqr[i] = 0.f;
#pragma unroll
  for (int hf = 0; hf < L::NH; ++hf)
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      float fk[8], fq[8];
      if constexpr (sizeof(T) == 2) {
        const uint4 a = kv[hf][i].a, b = qv[hf][i].a;
        fk[0] = bf16_lo(a.x); fk[1] = bf16_hi(a.x); fk[2] = bf16_lo(a.y); fk[3] = bf16_hi(a.y);
        fk[4] = bf16_lo(a.z); fk[5] = bf16_hi(a.z); fk[6] = bf16_lo(a.w); fk[7] = bf16_hi(a.w);
        fq[0] = bf16_lo(b.x); fq[1] = bf16_hi(b.x); fq[2] = bf16_lo(b.y); fq[3] = bf16_hi(b.y);
        fq[4] = bf16_lo(b.z); fq[5] = bf16_hi(b.z); fq[6] = bf16_lo(b.w); fq[7] = bf16_hi(b.w);
      } else {
        const uint4 a0 = kv[hf][i].a, a1 = kv[hf][i].b, b0 = qv[hf][i].a, b1 = qv[hf][i].b;
        fk[0] = __uint_as_float(a0.x); fk[1] = __uint_as_float(a0.y); fk[2] = __uint_as_float(a0.z);
        fk[3] = __uint_as_float(a0.w); fk[4] = __uint_as_float(a1.x); fk[5] = __uint_as_float(a1.y);
        fk[6] = __uint_as_float(a1.z); fk[7] = __uint_as_float(a1.w);
        fq[0] = __uint_as_float(b0.x); fq[1] = __uint_as_float(b0.y); fq[2] = __uint_as_float(b0.z);
        fq[3] = __uint_as_float(b0.w); fq[4] = __uint_as_float(b1.x); fq[5] = __uint_as_float(b1.y);
        fq[6] = __uint_as_float(b1.z); fq[7] = __uint_as_float(b1.w);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) { skr[i] += fk[j] * fk[j]; sqr[i] += fq[j] * fq[j]; }
    }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    float sk = skr[i], sq = sqr[i];
    sk += dpp_f32<DPP_QUAD_1032>(sk); sk += dpp_f32<DPP_QUAD_2301>(sk);
    sq += dpp_f32<DPP_QUAD_1032>(sq); sq += dpp_f32<DPP_QUAD_2301>(sq);
    if constexpr (RTH >= 8) { sk += dpp_f32<DPP_ROW_HALF_MIRROR>(sk); sq += dpp_f32<DPP_ROW_HALF_MIRROR>(sq); }
    if constexpr (RTH == 16) { sk += dpp_f32<DPP_ROW_MIRROR>(sk); sq += dpp_f32<DPP_ROW_MIRROR>(sq); }
    const int e = tid + i * NTH;
    if (e >= C * RTH) continue;  // a pass wider than the chunk (whole rows per pass)
    if (e % RTH == 0) {
      rk_s[e / RTH] = p.l2norm ? 1.0f / sqrtf(sk + 1e-6f) : 1.0f;
      rq_s[e / RTH] = p.l2norm ? 1.0f / sqrtf(sq + 1e-6f) : 1.0f;
    }
  }
  // raw rows into the swizzled tiles, d_k part hf of NH (rows >= Lc zero)
  auto stage = [&](int hf) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = tid + i * NTH;
      const int r = e / RTH, c0 = (e % RTH) * 8;
      if (e >= C * RTH) continue;
#pragma unroll
      for (int part = 0; part < (int)sizeof(R8) / 16; ++part) {
        const int b = c0 * (int)sizeof(T) + 16 * part;
        const uint4 zk = r < Lc ? (part ? reinterpret_cast<const uint4*>(&kv[hf][i])[1] : kv[hf][i].a) : make_uint4(0u, 0u, 0u, 0u);
        const uint4 zq = r < Lc ? (part ? reinterpret_cast<const uint4*>(&qv[hf][i])[1] : qv[hf][i].a) : make_uint4(0u, 0u, 0u, 0u);
        *reinterpret_cast<uint4*>(K_s + SK::off(r, b)) = zk;
        *reinterpret_cast<uint4*>(Q_s + SK::off(r, b)) = zq;
      }
    }
  };
  stage(0);
  if (ttid < C) {
    g_s[ttid] = ttid < Lc ? gv : 0.f;
    b_s[ttid] = ttid < Lc ? bv : 0.f;
  }
  __syncthreads();

  // cumulative log-decay over the chunk
  if (wave == 0) {
    float G = lane < C ? g_s[lane] : 0.f;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float u = __shfl_up(G, o, 64);
      if (lane >= o) G += u;
    }
    if (lane < C) G_s[lane] = G;
  }
  // transposed Gram tiles below the diagonal: job (mt, tj), tj <= mt, holds
  // rows j = 16 tj + 4g + i, column r = 16 mt + l16 of K K^T (jobs
  // [0, NLT)) or of K Q^T (jobs [NLT, 2 NLT)).  jmt/jnt: a team wave's
  // masked jobs (wave + 4 jj); gmt/gnt: its Gram jobs (gwave + GW jj), the
  // same ones unless the teams share the tiles.
  auto job_tile = [](int job, int& mt, int& tj) {
    tj = job >= NLT ? job - NLT : job;
    mt = 0;
    while (tj > mt) { tj -= mt + 1; ++mt; }
  };
  const int gwave = L::share ? tid >> 6 : wave;
  f32x4 gram[NJG];
  int jmt[NJ], jnt[NJ], gmt[NJG], gnt[NJG];
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj) {
    const int job = wave + 4 * jj;
    jmt[jj] = jnt[jj] = 0;
    if (job < 2 * NLT) job_tile(job, jmt[jj], jnt[jj]);
  }
#pragma unroll
  for (int jj = 0; jj < NJG; ++jj) {
    const int job = gwave + GW * jj;
    gram[jj] = f32x4{0.f, 0.f, 0.f, 0.f};
    gmt[jj] = gnt[jj] = 0;
    if (job < 2 * NLT) job_tile(job, gmt[jj], gnt[jj]);
  }
  // the k-steps over the staged part of d_k
  auto gram_pass = [&]() {
#pragma unroll
    for (int jj = 0; jj < NJG; ++jj) {
      const int job = gwave + GW * jj;
      if (job < 2 * NLT) {
        const unsigned char* Bt = job >= NLT ? Q_s : K_s;
#pragma unroll
        for (int s = 0; s < L::DH / 32; ++s)
          M::mma(gram[jj], frag_row<T, L::RBH>(K_s, gnt[jj] * 16 + l16, 32 * s + 8 * g4, false),
                 frag_row<T, L::RBH>(Bt, gmt[jj] * 16 + l16, 32 * s + 8 * g4, false), false);
      }
    }
  };
  gram_pass();
  if constexpr (L::NH == 2) {
    __syncthreads();  // the first half is read
    stage(1);
    __syncthreads();
    gram_pass();
  }
  if constexpr (L::share) {  // the raw tiles, for every team's masks
#pragma unroll
    for (int jj = 0; jj < NJG; ++jj) {
      const int job = gwave + GW * jj;
      if (job < 2 * NLT) *reinterpret_cast<f32x4*>(smem + L::oStage + job * 1024 + lane * 16) = gram[jj];
    }
  }
  __syncthreads();  // norms, G and the tiles published; K, Q are dead from here on

  unsigned char* rec = ws + off_bytes(p.n_seqs) + ((size_t)ci * p.h_v + h) * Rec<T, C>::bytes;
  T* Tb_g = reinterpret_cast<T*>(rec);
  T* P_g = reinterpret_cast<T*>(rec + Rec<T, C>::mat);
  float* vec_g = reinterpret_cast<float*>(rec + 2 * Rec<T, C>::mat);
  if (ttid < C) {
    const float G = G_s[ttid], Gl = G_s[Lc - 1], eg = fexp(G);
    vec_g[ttid] = p.erase ? eg * rk_s[ttid] : 0.f;  // no erase: R = V
    vec_g[C + ttid] = p.scale * eg * rq_s[ttid];
    vec_g[2 * C + ttid] = fexp(Gl - G) * rk_s[ttid];
    vec_g[3 * C + ttid] = fexp(Gl);
  }
  // decay-masked tiles: A (strict lower, fp32, to LDS) and P (lower incl.
  // the diagonal, to the workspace); a lane holds row r, columns j0..j0+3
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj) {
    const int job = wave + 4 * jj;
    if (job < 2 * NLT) {
      const bool isP = job >= NLT;
      const int r = jmt[jj] * 16 + l16, j0 = jnt[jj] * 16 + 4 * g4;
      // row factor (scale rq_r for P, beta_r rk_r for A, or 0 for A without
      // the erase: T = I) and the four columns' G and rk, each read once
      const float Gr = G_s[r];
      const float fr = isP ? p.scale * rq_s[r] : p.erase ? b_s[r] * rk_s[r] : 0.f;
      const float4 Gj = *reinterpret_cast<const float4*>(G_s + j0);
      const float4 kj = *reinterpret_cast<const float4*>(rk_s + j0);
      const float gj[4] = {Gj.x, Gj.y, Gj.z, Gj.w}, rkj[4] = {kj.x, kj.y, kj.z, kj.w};
      f32x4 gt;
      if constexpr (L::share) gt = *reinterpret_cast<const f32x4*>(smem + L::oStage + job * 1024 + lane * 16);
      else gt = gram[jj];
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = j0 + i;
        const bool keep = isP ? j <= r : j < r;
        v[i] = keep ? fr * fexp(Gr - gj[i]) * rkj[i] * gt[i] : 0.f;
      }
      if (isP) {
        if constexpr (sizeof(T) == 2)
          *reinterpret_cast<uint2*>(P_g + r * C + j0) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        else
          *reinterpret_cast<float4*>(P_g + r * C + j0) = make_float4(v[0], v[1], v[2], v[3]);
      } else {
        *reinterpret_cast<float4*>(A_s + r * L::LDF + j0) = make_float4(v[0], v[1], v[2], v[3]);
      }
    }
  }
  // P above the diagonal tiles is zero
  constexpr int NUP = NT * (NT - 1) / 2 * 16 * 16 / 8;  // 8-element pieces of the upper tiles
  for (int e = ttid; e < NUP; e += kPrepThreads) {
    int k = e / 32, mt = 0;  // tile k of the upper tiles, row-major (mt, tj > mt)
    while (k >= NT - 1 - mt) { k -= NT - 1 - mt; ++mt; }
    const int tj = mt + 1 + k, rr = (e % 32) / 2, half = e % 2;
    R8::zero().store(P_g + (mt * 16 + rr) * C + tj * 16 + 8 * half);
  }
  __syncthreads();

  // T = (I + A)^-1 by 16x16 blocks, in place: the diagonal blocks by forward
  // substitution, the blocks below them on fp32 MFMA.  A block X of
  // A_s is read as the accumulator layout of X (col: lane (g, c) holds
  // X[4g+i][c]) or of X^T (row: X[c][4g+i], one 16-byte read); tn(Y, W)
  // forms Y^T W from two such tiles.
  const int c16 = lane & 15;
  auto col = [&](int bi, int bj) {
    const float* a = A_s + (16 * bi + 4 * g4) * L::LDF + 16 * bj + c16;
    return f32x4{a[0], a[L::LDF], a[2 * L::LDF], a[3 * L::LDF]};
  };
  auto row = [&](int bi, int bj) {
    const float4 v = *reinterpret_cast<const float4*>(A_s + (16 * bi + c16) * L::LDF + 16 * bj + 4 * g4);
    return f32x4{v.x, v.y, v.z, v.w};
  };
  auto put = [&](int bi, int bj, const f32x4& t, float sgn) {
    float* a = A_s + (16 * bi + 4 * g4) * L::LDF + 16 * bj + c16;
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i * L::LDF] = sgn * t[i];
  };
  // diagonal blocks: wave 0 inverts each unit lower-triangular I + N (N the
  // strictly lower 16x16 block) by forward substitution in fp32, lane
  // (b, k) = (lane / 16, lane % 16) forming column k of block b:
  // t_i = [i == k] - sum_{j < i} N_ij t_j (zero above k, one at k).  Rows of
  // N are read as broadcasts (the 16 lanes of a block share each address).
  if (wave == 0 && (lane >> 4) < NT) {
    const int b = lane >> 4, k = lane & 15;
    const float* nb = A_s + 16 * b * L::LDF + 16 * b;  // block (b, b)
    float t[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float acc = i == k ? 1.f : 0.f;
#pragma unroll
      for (int q = 0; q < (i + 3) / 4; ++q) {
        const float4 n4 = *reinterpret_cast<const float4*>(nb + i * L::LDF + 4 * q);
        const float nv[4] = {n4.x, n4.y, n4.z, n4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (4 * q + e < i) acc -= nv[e] * t[4 * q + e];
      }
      t[i] = acc;
    }
    float* out = A_s + 16 * b * L::LDF + 16 * b + k;
#pragma unroll
    for (int i = 0; i < 16; ++i) out[i * L::LDF] = t[i];
  }
  __syncthreads();
  if constexpr (NT >= 2) {
    // level 1: T_{2b+1,2b} = -T_{2b+1,2b+1} A_{2b+1,2b} T_{2b,2b}
    if (wave < NT && (wave & 1) == 0) {
      const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
      const f32x4 z1 = mfma_tn(row(wave + 1, wave), col(wave, wave), zero);  // A_{2b+1,2b} T_{2b,2b}
      put(wave + 1, wave, mfma_tn(row(wave + 1, wave + 1), z1, zero), -1.f);
    }
    __syncthreads();
  }
  if constexpr (NT == 4) {
    // level 2: T_[23][01] = -T_[23][23] Z with Z = A_[23][01] T_[01][01];
    // wave (i, j) = (2 + wave/2, wave%2) forms block (i, j), the i = 3 waves
    // recomputing the Z_2j they share
    const int j = wave & 1, i = 2 + (wave >> 1);
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    f32x4 t = zero;
    if (wave < 4) {
      const f32x4 T1j = col(1, j);
      f32x4 z2 = mfma_tn(row(2, 1), T1j, zero);
      if (j == 0) z2 = mfma_tn(row(2, 0), col(0, 0), z2);
      if (i == 2) {
        t = mfma_tn(row(2, 2), z2, zero);
      } else {
        f32x4 z3 = mfma_tn(row(3, 1), T1j, zero);
        if (j == 0) z3 = mfma_tn(row(3, 0), col(0, 0), z3);
        t = mfma_tn(row(3, 2), z2, zero);
        t = mfma_tn(row(3, 3), z3, t);
      }
    }
    __syncthreads();  // every A_[23][01] block read before any is replaced
    if (wave < 4) put(i, j, t, -1.f);
    __syncthreads();
  }

  // Tb = T diag(beta) (upper blocks zero), 8 consecutive elements of a row
  // per thread, straight to the workspace
  for (int e = ttid; e < C * C / 8; e += kPrepThreads) {
    const int r = e / (C / 8), j0 = (e % (C / 8)) * 8;
    float v[8];
    if ((j0 >> 4) > (r >> 4)) {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.f;
    } else {
      const float4 a0 = *reinterpret_cast<const float4*>(A_s + r * L::LDF + j0);
      const float4 a1 = *reinterpret_cast<const float4*>(A_s + r * L::LDF + j0 + 4);
      const float4 b0 = *reinterpret_cast<const float4*>(b_s + j0);
      const float4 b1 = *reinterpret_cast<const float4*>(b_s + j0 + 4);
      v[0] = a0.x * b0.x; v[1] = a0.y * b0.y; v[2] = a0.z * b0.z; v[3] = a0.w * b0.w;
      v[4] = a1.x * b1.x; v[5] = a1.y * b1.y; v[6] = a1.z * b1.z; v[7] = a1.w * b1.w;
    }
    store8(Tb_g + r * C + j0, v);
  }
}

// ------------------------------------------------------------------ scan
template <typename T, int D, int C, int NW, int CT>
struct ScanLayout {
  static constexpr int NT = C / 16;
  static constexpr int DT = D / 16;
  static constexpr int E = (int)sizeof(T);
  static constexpr int threads = 64 * NW;
  static constexpr int cols = 16 * CT * NW;
  static constexpr int RBK = D * E;     // K, Q rows
  static constexpr int RBC = C * E;     // Tb, P rows
  static constexpr int RBV = cols * E;  // V rows (this workgroup's columns)
  static constexpr int oK = 0;
  static constexpr int oQ = oK + C * RBK;
  static constexpr int oTb = oQ + C * RBK;
  static constexpr int oP = oTb + C * RBC;
  static constexpr int oV = oP + C * RBC;
  static constexpr int oVec = oV + C * RBV;
  static constexpr int buf = oVec + 16 * C;
  static constexpr int PADO = 16 / E;
  static constexpr int LDO = cols + PADO;  // O staging rows [token][cols]
  static constexpr int obuf = C * LDO * E;
  // Two chunk buffers (the next chunk lands while this one is computed) when
  // they fit in LDS; otherwise (fp32 at chunk 64) one, loaded between chunks.
  static constexpr int nbuf = 2 * buf <= 160 * 1024 ? 2 : 1;
  // O leaves through the staging tiles when they fit in LDS as well;
  // otherwise each lane stores its elements.
  static constexpr bool stage_o = nbuf * buf + 2 * obuf <= 160 * 1024;
  static constexpr int bytes = nbuf * buf + (stage_o ? 2 * obuf : 0);
  static constexpr int NOV = (C * cols / 8 + threads - 1) / threads;  // O vectors per thread
};

template <typename T, int D, int C, int NW, int CT>
__global__ __launch_bounds__(64 * NW) void scan_kernel(PrefillParams p, const unsigned char* ws) {
  using L = ScanLayout<T, D, C, NW, CT>;
  using M = Mma<T>;
  using frag = typename M::frag;
  constexpr int NT = L::NT, DT = L::DT;
  constexpr int NB = D / L::cols;  // column blocks per V head
  // Two chunk buffers and two O staging tiles as separate LDS objects: the
  // compiler can then see that the next chunk's direct-to-LDS loads never
  // touch what the current chunk reads, and inserts no wait for them.
  __shared__ __align__(16) unsigned char sb0[L::buf];
  __shared__ __align__(16) unsigned char sb1[L::nbuf == 2 ? L::buf : 16];
  __shared__ __align__(16) unsigned char so0[L::stage_o ? L::obuf : 16];
  __shared__ __align__(16) unsigned char so1[L::stage_o ? L::obuf : 16];
  // with one chunk buffer, every chunk is computed from sb0
  unsigned char* const sbn = L::nbuf == 2 ? sb1 : sb0;

  const PlanView pv = plan_view(p, ws, C);
  const ScanSlot slot = scan_slot(p, pv, NB);
  if (!slot.valid) return;
  const int blk = slot.blk, h = slot.h, n = slot.n;
  const int hq = h / (p.h_v / p.h_qk);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = lane >> 4, l16 = lane & 15;
  // this lane's column in the workgroup block for column tile ct
  auto lcol = [&](int ct) { return (wave * CT + ct) * 16 + l16; };

  const unsigned char* recs = ws + off_bytes(p.n_seqs);
  const int64_t seq_start = p.cu_seqlens ? p.cu_seqlens[n] : 0;
  const int64_t seq_end = p.cu_seqlens ? p.cu_seqlens[n + 1] : p.total_tokens;
  const int c0 = pv.off(n);
  const int nch = pv.off(n + 1) - c0;

  const unsigned char* qg = reinterpret_cast<const unsigned char*>(reinterpret_cast<const T*>(p.q) + (int64_t)hq * D);
  const unsigned char* kg = reinterpret_cast<const unsigned char*>(reinterpret_cast<const T*>(p.k) + (int64_t)hq * D);
  const unsigned char* vg = reinterpret_cast<const unsigned char*>(reinterpret_cast<const T*>(p.v) + (int64_t)h * D +
                                                                   blk * L::cols);
  const int64_t o_stride = (int64_t)p.h_v * D;
  T* og_blk = reinterpret_cast<T*>(p.o) + (int64_t)h * D + blk * L::cols;

  // direct-to-LDS loads of chunk c into `b`; rows past a partial chunk
  // re-read its last row: they only ever meet zero columns of Tb and zero
  // rows of U (beta = 0 there), so any finite values are harmless
  auto issue = [&](int c, unsigned char* b) {
    const int64_t t0 = seq_start + (int64_t)c * C;
    const int Lc = (int)min((int64_t)C, seq_end - t0);
    const unsigned char* rec = recs + ((size_t)(c0 + c) * p.h_v + h) * Rec<T, C>::bytes;
    dma_tile<L::RBK, C, NW>(b + L::oK, kg + t0 * p.k_stride * L::E, p.k_stride * L::E, Lc, wave, lane);
    dma_tile<L::RBK, C, NW>(b + L::oQ, qg + t0 * p.q_stride * L::E, p.q_stride * L::E, Lc, wave, lane);
    dma_tile<L::RBC, C, NW>(b + L::oTb, rec, L::RBC, C, wave, lane);
    dma_tile<L::RBC, C, NW>(b + L::oP, rec + Rec<T, C>::mat, L::RBC, C, wave, lane);
    dma_tile<L::RBV, C, NW>(b + L::oV, vg + t0 * p.v_stride * L::E, p.v_stride * L::E, Lc, wave, lane);
    dma_linear<16 * C, NW>(b + L::oVec, rec + 2 * Rec<T, C>::mat, wave, lane);
  };
  // O rows of chunk c leave the staging tile in 16-byte row pieces
  auto store_o = [&](const unsigned char* so, int64_t t0, int Lc) {
    const T* Ot = reinterpret_cast<const T*>(so);
#pragma unroll
    for (int i = 0; i < L::NOV; ++i) {
      const int e = tid + i * L::threads;
      const int r = e / (L::cols / 8), c8 = (e % (L::cols / 8)) * 8;
      if (e < C * L::cols / 8 && r < Lc)
        Raw8<T>::load(Ot + r * L::LDO + c8).store(og_blk + (t0 + r) * o_stride + c8);
    }
  };
  // per-token scalars of tile mt, rows 4g..4g+3: four consecutive tokens
  auto vec4 = [&](const float* v, int mt) { return *reinterpret_cast<const float4*>(v + pidx<NT>(mt, 4 * g4)); };

  // state S^T (d_k x 16 columns per column tile) in DT accumulator tiles;
  // row 4g+i of tile dt is d_k index pidx<DT>(dt, 4g+i)
  f32x4 st[CT][DT];
  const int sslot = p.state_idx ? as_const(p.state_idx)[n] : n;
  const size_t sbase = ((size_t)sslot * p.h_v + h) * D * D + (size_t)(blk * L::cols) * D;
  // rows of this sequence's emitted chunk-boundary states
  const int erow = p.emit_every > 0 ? pv.erow(n) : 0;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      st[ct][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (p.initial_state)
        st[ct][dt] = load_state4(p.initial_state, sbase + (size_t)lcol(ct) * D + pidx<DT>(dt, 4 * g4), p.state_bf16);
    }

  // one chunk: store the previous chunk's O, start the next chunk's loads
  // into `nxt`, compute this chunk from `cur`, stage its O in `ocur`
  auto step = [&](int c, const unsigned char* cur, unsigned char* nxt, unsigned char* ocur,
                  const unsigned char* oprev) {
    const int64_t t0 = seq_start + (int64_t)c * C;
    const unsigned char* K_t = cur + L::oK;
    const unsigned char* Q_t = cur + L::oQ;
    const unsigned char* Tb_t = cur + L::oTb;
    const unsigned char* P_t = cur + L::oP;
    const unsigned char* V_t = cur + L::oV;
    const float* vec = reinterpret_cast<const float*>(cur + L::oVec);
    if constexpr (L::stage_o) {
      if (c > 0) store_o(oprev, t0 - C, C);
    }
    if (L::nbuf == 2 && c + 1 < nch) issue(c + 1, nxt);
    constexpr int KS = (NT + 1) / 2;  // k-steps over the chunk's tokens
    constexpr bool HALF = NT == 1;    // a 16-token chunk: half-empty k-step

    // X1 = K S^T, Y = Q S^T: each K/Q fragment feeds every column tile
    f32x4 x1[CT][NT], yq[CT][NT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int mt = 0; mt < NT; ++mt) { x1[ct][mt] = f32x4{0.f, 0.f, 0.f, 0.f}; yq[ct][mt] = x1[ct][mt]; }
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      frag bs[CT], ak[NT], aq[NT];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) bs[ct] = M::acc(st[ct][2 * s], st[ct][2 * s + 1]);
#pragma unroll
      for (int mt = 0; mt < NT; ++mt) {
        const int row = pidx<NT>(mt, l16);
        ak[mt] = frag_row<T, L::RBK>(K_t, row, 32 * s + 8 * g4, false);
        aq[mt] = frag_row<T, L::RBK>(Q_t, row, 32 * s + 8 * g4, false);
      }
#pragma unroll
      for (int mt = 0; mt < NT; ++mt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          M::mma(x1[ct][mt], ak[mt], bs[ct], false);
          M::mma(yq[ct][mt], aq[mt], bs[ct], false);
        }
    }
    // R = V - diag(gamma rk) X1   (in place in x1)
#pragma unroll
    for (int mt = 0; mt < NT; ++mt) {
      const float4 vq = vec4(vec, mt);
      const float vs[4] = {vq.x, vq.y, vq.z, vq.w};
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = pidx<NT>(mt, 4 * g4 + i);
          const float vv = to_f32(*reinterpret_cast<const T*>(V_t + Swz<L::RBV>::off(r, lcol(ct) * L::E)));
          x1[ct][mt][i] = vv - vs[i] * x1[ct][mt][i];
        }
    }
    // U = Tb R
    f32x4 u[CT][NT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int mt = 0; mt < NT; ++mt) u[ct][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      frag bs[CT], at[NT];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) bs[ct] = M::acc(x1[ct][2 * s], tile_hi<NT>(x1[ct], s));
#pragma unroll
      for (int mt = 0; mt < NT; ++mt)
        at[mt] = frag_row<T, L::RBC>(Tb_t, pidx<NT>(mt, l16), HALF ? 4 * g4 : 32 * s + 8 * g4, HALF);
#pragma unroll
      for (int mt = 0; mt < NT; ++mt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) M::mma(u[ct][mt], at[mt], bs[ct], HALF);
    }
    // O = diag(scale gamma rq) Y + P U
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int mt = 0; mt < NT; ++mt) x1[ct][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      frag bs[CT], ap[NT];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) bs[ct] = M::acc(u[ct][2 * s], tile_hi<NT>(u[ct], s));
#pragma unroll
      for (int mt = 0; mt < NT; ++mt)
        ap[mt] = frag_row<T, L::RBC>(P_t, pidx<NT>(mt, l16), HALF ? 4 * g4 : 32 * s + 8 * g4, HALF);
#pragma unroll
      for (int mt = 0; mt < NT; ++mt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) M::mma(x1[ct][mt], ap[mt], bs[ct], HALF);
    }
#pragma unroll
    for (int mt = 0; mt < NT; ++mt) {
      const float4 vq = vec4(vec + C, mt);
      const float vs[4] = {vq.x, vq.y, vq.z, vq.w};
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        if constexpr (L::stage_o) {
          T* Ot = reinterpret_cast<T*>(ocur) + lcol(ct);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            Ot[pidx<NT>(mt, 4 * g4 + i) * L::LDO] = from_f32<T>(x1[ct][mt][i] + vs[i] * yq[ct][mt][i]);
        } else {
          const int Lc = (int)min((int64_t)C, seq_end - t0);
          T* og = og_blk + lcol(ct);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = pidx<NT>(mt, 4 * g4 + i);
            if (r < Lc) og[(t0 + r) * o_stride] = from_f32<T>(x1[ct][mt][i] + vs[i] * yq[ct][mt][i]);
          }
        }
      }
    }
    // S^T <- gamma_last S^T + K^T diag(e rk) U: each K^T fragment feeds every column tile
    const float gl = vec[3 * C];
#pragma unroll
    for (int mt = 0; mt < NT; ++mt) {
      const float4 vq = vec4(vec + 2 * C, mt);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        u[ct][mt][0] *= vq.x; u[ct][mt][1] *= vq.y; u[ct][mt][2] *= vq.z; u[ct][mt][3] *= vq.w;
      }
    }
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) st[ct][dt] *= gl;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      frag bs[CT];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) bs[ct] = M::acc(u[ct][2 * s], tile_hi<NT>(u[ct], s));
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const frag ak = frag_kt<T, L::RBK, DT>(K_t, dt, HALF ? 4 * g4 : 32 * s + 8 * g4, l16, HALF);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) M::mma(st[ct][dt], ak, bs[ct], HALF);
      }
    }
    // the state after every emit_every-th whole chunk inside the sequence
    if (p.emit_every > 0 && (c + 1) % p.emit_every == 0 && t0 + C < seq_end) {
      const size_t dst = ((size_t)(erow + (c + 1) / p.emit_every - 1) * p.h_v + h) * D * D +
                         (size_t)(blk * L::cols) * D;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          store_state4(p.chunk_states, dst + (size_t)lcol(ct) * D + pidx<DT>(dt, 4 * g4), st[ct][dt], p.state_bf16);
    }
    __syncthreads();  // waits for the next chunk's loads; frees `cur`
    if (L::nbuf == 1 && c + 1 < nch) {
      issue(c + 1, nxt);  // nxt == cur: every read of this chunk is done
      __syncthreads();
    }
  };

  if (nch > 0) issue(0, sb0);
  __syncthreads();  // waits for the loads of chunk 0
  for (int c = 0; c < nch; c += 2) {
    step(c, sb0, sbn, so0, so1);
    if (c + 1 < nch) step(c + 1, sbn, sb0, so1, so0);
  }
  if (L::stage_o && nch > 0) {
    const int64_t tl = seq_start + (int64_t)(nch - 1) * C;
    store_o(((nch - 1) & 1) ? so1 : so0, tl, (int)(seq_end - tl));
  }

  if (p.final_state) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        store_state4(p.final_state, sbase + (size_t)lcol(ct) * D + pidx<DT>(dt, 4 * g4), st[ct][dt], p.state_bf16);
  }
}

// ------------------------------------------------------- split-role scan
// bf16 scan with three wave roles per workgroup, for a block of 32 or 64 d_v
// columns of one (sequence, V head):
//  chain waves (one per 16 columns) own their columns of the fp32 state S^T
//    in accumulator tiles and run the serial part of a chunk:  X1 = K S^T,
//    R = V - diag(gamma rk) X1,  U = Tb R,  S^T <- gamma_last S^T + K^T diag(e rk) U;
//  output waves (two per 16 columns, each on half of the chunk's tokens)
//    compute the chunk's output O^T = (S Q^T) diag(scale gamma rq) + U^T P^T
//    from the state and U that the chain waves publish in LDS as bf16, and
//    store O straight from their accumulators (a lane holds 4 consecutive
//    columns of one token);
//  mover waves (32-column workgroups only) issue the next chunk's
//    direct-to-LDS loads and the L2 prefetch; without them the output waves
//    issue the loads.
// Waves are placed on SIMDs by role (see the kernel).  Per chunk: barrier B1
// once U is published and the chain has updated its registers (LDS only: the
// loads stay in flight), and B2 at the end (the next chunk has landed, the
// new state is published).
template <int D, int C, int COLS>
struct Scan2Layout {
  static constexpr int NT = C / 16, DT = D / 16;
  static constexpr int cols = COLS;  // d_v columns per workgroup
  static constexpr int RBK = D * 2, RBC = C * 2, RBV = cols * 2, RBS = D * 2, RBU = C * 2;
  using SK = Swz<RBK>;
  using SC = Swz<RBC>;
  using SV = SwzT<RBV, RowV<NT, RBV / 16>>;
  using SS = SwzT<RBS, RowSeq<RBS>>;
  using SU = SwzT<RBU, RowSeq<RBU>>;
  static constexpr int oK = 0;
  static constexpr int oQ = oK + C * RBK;
  static constexpr int oTb = oQ + C * RBK;
  static constexpr int oP = oTb + C * RBC;
  static constexpr int oV = oP + C * RBC;
  static constexpr int oVec = oV + C * RBV;
  static constexpr int buf = oVec + 16 * C;
  static constexpr int sbytes = cols * RBS;
  static constexpr int ubytes = cols * RBU;
  static constexpr int bytes = 2 * buf + sbytes + ubytes;
};

// s_waitcnt with vmcnt(vm), expcnt untouched, lgkmcnt(0)
template <int VM>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4));
}
// Workgroup barrier that waits only for what is named: this wave's LDS
// operations and all but its last VM vector-memory operations.
template <int VM>
__device__ __forceinline__ void barrier_vm() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  wait_vm_lgkm0<VM>();
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

template <int D, int C, int CT, int NWR, int OS, int NM>
__global__ __launch_bounds__(64 * (NWR * (1 + OS) + NM)) void scan2_kernel(PrefillParams p, const unsigned char* ws,
                                                                          ScanSplit sp) {
  using L = Scan2Layout<D, C, 16 * CT * NWR>;
  using T = __bf16;
  using M = Mma<T>;
  using frag = typename M::frag;
  using SK = typename L::SK;
  using SC = typename L::SC;
  using SV = typename L::SV;
  using SS = typename L::SS;
  using SU = typename L::SU;
  constexpr int NT = L::NT, DT = L::DT, DKS = D / 32;
  constexpr int KS = (NT + 1) / 2;  // k-steps over the chunk's tokens
  constexpr bool HALF = NT == 1;    // a 16-token chunk: half-empty k-step
  constexpr int NB = D / L::cols;
  // NWR chain waves; OS output waves per chain wave's column slice, each
  // forming NT / OS of the chunk's 16-token tiles
  constexpr int SW = 16 * CT;       // columns per wave
  constexpr int NO = NWR * OS, NTO = NT / OS;
  static_assert(NT % OS == 0, "token tiles split evenly over the output waves of a slice");
  // NM mover waves (if any) issue the next chunk's loads; without them the
  // output waves do
  constexpr int NX = NM > 0 ? NM : NO;
  __shared__ __align__(16) unsigned char sb0[L::buf];
  __shared__ __align__(16) unsigned char sb1[L::buf];
  __shared__ __align__(16) unsigned char sS[L::sbytes];
  __shared__ __align__(16) unsigned char sU[L::ubytes];

  const PlanView plan = plan_view(p, ws, C);
  const ScanSlot slot = sp.on ? split_slot(p, NB) : scan_slot(p, plan, NB);
  if (!slot.valid) return;
  const int blk = slot.blk, h = slot.h, n = slot.n, role = slot.role;
  const int hq = h / (p.h_v / p.h_qk);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = lane >> 4, l16 = lane & 15;
  // Waves w and w + 4 of a workgroup share a SIMD.  With movers (eight
  // waves) the chain waves 0 .. NWR-1 share their SIMDs only with the movers
  // 4 .. 4+NWR-1, which issue loads and little else; the output waves take
  // the other two slots of the remaining SIMDs.  Without movers the output
  // waves follow the chain waves.
  static_assert(NM == 0 || (NM == NWR && NWR + NO / 2 == 4), "mover layout: eight waves, two per SIMD");
  const int slot4 = wave & 3, hi4 = wave >> 2;
  const bool chain = NM > 0 ? (slot4 < NWR && hi4 == 0) : wave < NWR;
  const bool mover = NM > 0 && slot4 < NWR && hi4 == 1;
  const int ow = chain || mover ? 0 : NM > 0 ? slot4 - NWR + (4 - NWR) * hi4 : wave - NWR;  // index among the output waves
  const int cw = chain ? slot4 : ow % NWR;           // column slice: columns SW cw .. SW cw + SW - 1
  const int th = chain ? 0 : ow / NWR;               // output waves: token tiles [th NTO, (th + 1) NTO)
  const bool moves = NM > 0 ? mover : !chain;        // issues the loads of chunks 1, 2, ...
  const int xw = NM > 0 ? (mover ? slot4 : 0) : ow;  // index among the moving waves
  auto colof = [&](int ct) { return SW * cw + 16 * ct + l16; };  // this lane's column in tile ct

  const unsigned char* recs = ws + off_bytes(p.n_seqs);
  const int64_t seq_start = p.cu_seqlens ? p.cu_seqlens[n] : 0;
  const int64_t seq_end = p.cu_seqlens ? p.cu_seqlens[n + 1] : p.total_tokens;
  // this workgroup's chunks: the whole sequence, or one segment of a split
  const int cseq = plan.off(n), nch_seq = plan.off(n + 1) - cseq;
  const int cbeg = role == 0 ? 0 : sp.m;
  const int nch = sp.on ? (role == 0 ? sp.m : nch_seq - sp.m) : nch_seq;
  const int c0 = cseq + cbeg;
  const int64_t seg_start = seq_start + (int64_t)cbeg * C;

  const unsigned char* qg = reinterpret_cast<const unsigned char*>(reinterpret_cast<const T*>(p.q) + (int64_t)hq * D);
  const unsigned char* kg = reinterpret_cast<const unsigned char*>(reinterpret_cast<const T*>(p.k) + (int64_t)hq * D);
  // the transition role scans zero values: every V row reads the zero line
  const int64_t vrow = role == 2 ? 0 : p.v_stride * 2;
  const unsigned char* vg =
      role == 2 ? g_zero_line
                : reinterpret_cast<const unsigned char*>(reinterpret_cast<const T*>(p.v) + (int64_t)h * D + blk * L::cols);
  auto chunk_t0 = [&](int c) { return seg_start + (int64_t)c * C; };
  auto chunk_len = [&](int c) { return (int)min((int64_t)C, seq_end - chunk_t0(c)); };
  auto chunk_rec = [&](int c) { return recs + ((size_t)(c0 + c) * p.h_v + h) * Rec<T, C>::bytes; };

  // ---- data movement.  Chunk 0 is loaded by all waves before the roles
  // split; after that the mover waves (else the output waves) issue the next
  // chunk at the start of a chunk, so the loads have the whole chunk to land.
  // A wave that issues them stalls until the CU's load path has room, so with
  // movers neither the chain nor the output waves issue any load.  A full chunk uses per-lane offsets computed
  // once (DmaPlan); a partial chunk (the last of a sequence) takes the
  // clamped path, where rows past its end re-read its last row: they only
  // meet zero columns of Tb and zero rows of U.
  DmaPlan<SK, C, NX> pk, pq;
  DmaPlan<SC, C, NX> ptb;
  DmaPlan<SV, C, NX> pv;
  const bool fast = p.q_stride * 2 * C < (1ll << 31) && p.k_stride * 2 * C < (1ll << 31) &&
                    p.v_stride * 2 * C < (1ll << 31);
  if (fast && moves) {
    pk.init((uint32_t)(p.k_stride * 2), xw, lane);
    pq.init((uint32_t)(p.q_stride * 2), xw, lane);
    ptb.init((uint32_t)L::RBC, xw, lane);
    pv.init((uint32_t)vrow, xw, lane);
  }
  auto chunk_ptrs = [&](int c, const unsigned char*& kc, const unsigned char*& qc, const unsigned char*& vc,
                        const unsigned char*& rec) {
    const int64_t t0 = chunk_t0(c);
    kc = kg + t0 * p.k_stride * 2;
    qc = qg + t0 * p.q_stride * 2;
    vc = vg + t0 * vrow;
    rec = chunk_rec(c);
  };
  // clamped (any chunk), over NW waves with wave index w
  auto issue_slow = [&](int c, unsigned char* b, auto nw, int w) {
    constexpr int NW = decltype(nw)::value;
    const unsigned char *kc, *qc, *vc, *rec;
    chunk_ptrs(c, kc, qc, vc, rec);
    const int Lc = chunk_len(c);
    dma_tile_s<SK, C, NW>(b + L::oK, kc, p.k_stride * 2, Lc, w, lane);
    dma_tile_s<SK, C, NW>(b + L::oQ, qc, p.q_stride * 2, Lc, w, lane);
    dma_tile_s<SC, C, NW>(b + L::oTb, rec, L::RBC, C, w, lane);
    dma_tile_s<SC, C, NW>(b + L::oP, rec + Rec<T, C>::mat, L::RBC, C, w, lane);
    dma_tile_s<SV, C, NW>(b + L::oV, vc, vrow, Lc, w, lane);
    dma_linear<16 * C, NW>(b + L::oVec, rec + 2 * Rec<T, C>::mat, w, lane);
  };

  // the next chunk, c + 1, into nxt, by the moving waves
  auto issue_next = [&](int c, unsigned char* nxt) {
    if (c + 1 >= nch) return;
    if (fast && chunk_len(c + 1) == C) {
      const unsigned char *kc, *qc, *vc, *rec;
      chunk_ptrs(c + 1, kc, qc, vc, rec);
      pk.issue(nxt + L::oK, kc, xw, lane);
      pq.issue(nxt + L::oQ, qc, xw, lane);
      ptb.issue(nxt + L::oTb, rec, xw, lane);
      ptb.issue(nxt + L::oP, rec + Rec<T, C>::mat, xw, lane);
      pv.issue(nxt + L::oV, vc, xw, lane);
      dma_linear<16 * C, NX>(nxt + L::oVec, rec + 2 * Rec<T, C>::mat, xw, lane);
    } else {
      issue_slow(c + 1, nxt, std::integral_constant<int, NX>{}, xw);
    }
  };
  if (nch > 0) issue_slow(0, sb0, std::integral_constant<int, NWR + NO + NM>{}, wave);

  // L2 prefetch PFD chunks ahead, by the chain waves or the movers: one
  // 4-byte load per 128-byte line of the chunk's K, Q and V rows and of its
  // record, consumed a chunk later, so nothing waits for it.  The K, Q and
  // record lines, which the NB column blocks of a head share, are split
  // between the blocks.  Only the 32-column workgroups prefetch: they run
  // when the launch leaves CUs idle and the scan waits on HBM latency; with
  // every CU busy the extra requests cost more than they save.
  constexpr int PFD = L::cols == 32 ? 3 : 0;
  constexpr int TW = NM > 0 ? NM : NWR;  // touching waves
  constexpr int LPR = (D * 2 + 127) / 128;  // lines per K or Q row
  constexpr int NKL = C * LPR;
  constexpr int NSH = 2 * NKL + (int)(Rec<T, C>::bytes / 128);
  constexpr int NTOUCH = PFD > 0 ? ((NSH + NB - 1) / NB + C + 64 * TW - 1) / (64 * TW) : 0;
  const bool touches = PFD > 0 && (NM > 0 ? mover : chain);
  const int tw = NM > 0 ? xw : cw;
  // touch i of chunk c reads tbase[i] + c * tstep[i]
  const unsigned char* tbase[NTOUCH > 0 ? NTOUCH : 1];
  uint32_t tstep[NTOUCH > 0 ? NTOUCH : 1];
  uint32_t tv[NTOUCH > 0 ? NTOUCH : 1];
  const unsigned char* rec0 = chunk_rec(0);  // always a whole record
  if (touches) {
    const int nsw = (NSH - blk + NB - 1) / NB;  // shared lines of this block
    const int64_t ks = p.k_stride * 2, qs = p.q_stride * 2, vs = vrow;
#pragma unroll
    for (int i = 0; i < NTOUCH; ++i) {
      const int sl = (i * TW + tw) * 64 + lane;
      tv[i] = 0u;
      tbase[i] = rec0;
      tstep[i] = (uint32_t)(p.h_v * Rec<T, C>::bytes);
      if (sl < nsw) {
        const int l = blk + NB * sl;
        if (l < 2 * NKL) {
          const bool isq = l >= NKL;
          const int lk = isq ? l - NKL : l;
          const int64_t st = isq ? qs : ks;
          tbase[i] = (isq ? qg : kg) + seg_start * st + (lk / LPR) * st + (lk % LPR) * 128;
          tstep[i] = (uint32_t)(C * st);
        } else {
          tbase[i] = rec0 + (l - 2 * NKL) * 128;
        }
      } else if (sl < nsw + C) {
        tbase[i] = vg + seg_start * vs + (sl - nsw) * vs;
        tstep[i] = (uint32_t)(C * vs);
      }
    }
  }
  // the previous touches have landed; chunk c + PFD is touched (without a
  // full chunk c + PFD, every touch re-reads the sequence's first record)
  auto touch = [&](int c) {
#pragma unroll
    for (int i = 0; i < NTOUCH; ++i) asm volatile("" ::"v"(tv[i]));
    const bool ok = fast && c + PFD < nch && chunk_len(c + PFD) == C;
#pragma unroll
    for (int i = 0; i < NTOUCH; ++i)
      tv[i] = *reinterpret_cast<const uint32_t*>(ok ? tbase[i] + (uint64_t)(c + PFD) * tstep[i] : rec0);
  };

  if (chain) {
    // ---------------------------------------------------------- chain waves
    // state S^T (d_k x 16 columns) of column tile ct in DT accumulator
    // tiles; row 4g+i of tile dt is d_k index pidx<DT>(dt, 4g+i)
    f32x4 st[CT][DT];
    // row of this lane's column in the caller's state pools (slot of
    // sequence n) and in the split's workspace states (one sequence)
    const int sslot = p.state_idx ? as_const(p.state_idx)[n] : n;
    auto srow = [&](int ct) { return (((size_t)sslot * p.h_v + h) * D + (size_t)(blk * L::cols + colof(ct))) * D; };
    auto wrow = [&](int ct) { return ((size_t)h * D + (size_t)(blk * L::cols + colof(ct))) * D; };
    const int erow = p.emit_every > 0 ? plan.erow(n) : 0;
    // initial state: the caller's (or zero) for a whole sequence or a first
    // segment, zero for a second segment, the identity for the transition
    const void* s_init = role == 0 ? p.initial_state : nullptr;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        st[ct][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (s_init) st[ct][dt] = load_state4(s_init, srow(ct) + pidx<DT>(dt, 4 * g4), p.state_bf16);
        if (role == 2) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            st[ct][dt][i] = pidx<DT>(dt, 4 * g4 + i) == blk * L::cols + colof(ct) ? 1.f : 0.f;
        }
      }
    // the state as bf16 rows [column][d_k] for the output waves: tiles 2u,
    // 2u+1 give this lane d_k 32u + 8g .. 32u + 8g + 7
    auto publish_state = [&]() {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int u = 0; u < DT / 2; ++u)
          *reinterpret_cast<frag*>(sS + SS::off(colof(ct), (32 * u + 8 * g4) * 2)) =
              M::acc(st[ct][2 * u], st[ct][2 * u + 1]);
    };
    publish_state();
    __syncthreads();  // initial state published; chunk 0 has landed

    auto step = [&](int c, const unsigned char* cur) {
      const unsigned char* K_t = cur + L::oK;
      const unsigned char* Tb_t = cur + L::oTb;
      const unsigned char* V_t = cur + L::oV;
      const float* vec = reinterpret_cast<const float*>(cur + L::oVec);
      // operands of R and U that do not depend on the state, read up front:
      // V[token pidx(mt, 4g) + e][column] (one transposing read per tile) and Tb
      uint2 vw[CT][NT];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int mt = 0; mt < NT; ++mt) {
          const int r0 = pidx<NT>(mt, 4 * g4);
          vw[ct][mt] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(
              __attribute__((address_space(3))) unsigned char*)(V_t + SV::off(r0 + (l16 >> 2),
                                                                               (SW * cw + 16 * ct + 4 * (l16 & 3)) * 2))));
        }
      frag at[KS][NT];
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int mt = 0; mt < NT; ++mt)
          at[s][mt] = frag_row_s<T, SC>(Tb_t, pidx<NT>(mt, l16), HALF ? 4 * g4 : 32 * s + 8 * g4, HALF);
      // X1 = K S^T: each K fragment feeds every column tile
      f32x4 x1[CT][NT];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int mt = 0; mt < NT; ++mt) x1[ct][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < DKS; ++s) {
        frag bs[CT], ak[NT];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) bs[ct] = M::acc(st[ct][2 * s], st[ct][2 * s + 1]);
#pragma unroll
        for (int mt = 0; mt < NT; ++mt) ak[mt] = frag_row_s<T, SK>(K_t, pidx<NT>(mt, l16), 32 * s + 8 * g4, false);
#pragma unroll
        for (int mt = 0; mt < NT; ++mt)
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) M::mma(x1[ct][mt], ak[mt], bs[ct], false);
      }
      // K^T fragments of the state update, read while X1 drains
      frag kt[KS][DT];
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          kt[s][dt] = frag_kt<T, L::RBK, DT>(K_t, dt, HALF ? 4 * g4 : 32 * s + 8 * g4, l16, HALF);
      // R = V - diag(gamma rk) X1
#pragma unroll
      for (int mt = 0; mt < NT; ++mt) {
        const float4 vq = *reinterpret_cast<const float4*>(vec + pidx<NT>(mt, 4 * g4));
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          x1[ct][mt][0] = bf16_lo(vw[ct][mt].x) - vq.x * x1[ct][mt][0];
          x1[ct][mt][1] = bf16_hi(vw[ct][mt].x) - vq.y * x1[ct][mt][1];
          x1[ct][mt][2] = bf16_lo(vw[ct][mt].y) - vq.z * x1[ct][mt][2];
          x1[ct][mt][3] = bf16_hi(vw[ct][mt].y) - vq.w * x1[ct][mt][3];
        }
      }
      // U = Tb R
      f32x4 u[CT][NT];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int mt = 0; mt < NT; ++mt) u[ct][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        frag bs[CT];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) bs[ct] = M::acc(x1[ct][2 * s], tile_hi<NT>(x1[ct], s));
#pragma unroll
        for (int mt = 0; mt < NT; ++mt)
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) M::mma(u[ct][mt], at[s][mt], bs[ct], HALF);
      }
      // publish U as bf16 rows [column][token] (natural token order)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          if constexpr (HALF) {
            *reinterpret_cast<uint2*>(sU + SU::off(colof(ct), 8 * g4)) =
                make_uint2(pack_bf16x2(u[ct][0][0], u[ct][0][1]), pack_bf16x2(u[ct][0][2], u[ct][0][3]));
          } else {
            *reinterpret_cast<frag*>(sU + SU::off(colof(ct), (32 * s + 8 * g4) * 2)) =
                M::acc(u[ct][2 * s], u[ct][2 * s + 1]);
          }
        }
      // U' = diag(e rk) U for the state update
#pragma unroll
      for (int mt = 0; mt < NT; ++mt) {
        const float4 vq = *reinterpret_cast<const float4*>(vec + 2 * C + pidx<NT>(mt, 4 * g4));
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          u[ct][mt][0] *= vq.x; u[ct][mt][1] *= vq.y; u[ct][mt][2] *= vq.z; u[ct][mt][3] *= vq.w;
        }
      }
      const float gl = vec[3 * C];
      if (NM == 0 && touches) touch(c);
      // S^T <- gamma_last S^T + K^T diag(e rk) U in registers, before B1: the
      // state in LDS changes only after it
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) st[ct][dt] *= gl;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        frag bs[CT];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) bs[ct] = M::acc(u[ct][2 * s], tile_hi<NT>(u[ct], s));
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) M::mma(st[ct][dt], kt[s][dt], bs[ct], HALF);
      }
      barrier_vm<63>();  // B1: U is visible; the output waves are done with the old state
      // the state after every emit_every-th whole chunk inside the sequence
      // (a split scan never emits: its second segment does not hold S)
      if (p.emit_every > 0 && (cbeg + c + 1) % p.emit_every == 0 && chunk_t0(c) + C < seq_end) {
        const size_t dst = (size_t)(erow + (cbeg + c + 1) / p.emit_every - 1) * p.h_v * D * D;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
            store_state4(p.chunk_states, dst + wrow(ct) + pidx<DT>(dt, 4 * g4), st[ct][dt], p.state_bf16);
      }
      publish_state();
      __syncthreads();  // B2: next chunk loaded, new state published
    };
    for (int c = 0; c < nch; c += 2) {
      step(c, sb0);
      if (c + 1 < nch) step(c + 1, sb1);
    }
    if (NM == 0 && touches) {
#pragma unroll
      for (int i = 0; i < NTOUCH; ++i) asm volatile("" ::"v"(tv[i]));
    }
    // final state: the caller's, or the split's S_m (always: the join needs
    // it), S0 and Phi (only when the caller wants a final state)
    // (the split's states are internal fp32; the caller's in its state dtype)
    void* s_fin = !sp.on ? p.final_state
                : role == 0 ? (void*)sp.s_mid
                : !p.final_state ? nullptr
                : role == 1 ? (void*)sp.s_zero : (void*)sp.phi;
    const bool fin_bf16 = !sp.on && p.state_bf16;
    if (s_fin) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          store_state4(s_fin, (sp.on ? wrow(ct) : srow(ct)) + pidx<DT>(dt, 4 * g4), st[ct][dt], fin_bf16);
    }
    if (sp.on && role == 0) {  // S_m once more, as the join's bf16 operand
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          *reinterpret_cast<uint2*>(sp.s_mid_bf + wrow(ct) + pidx<DT>(dt, 4 * g4)) =
              make_uint2(pack_bf16x2(st[ct][dt][0], st[ct][dt][1]), pack_bf16x2(st[ct][dt][2], st[ct][dt][3]));
    }
  } else if (!mover) {
    // --------------------------------------------------------- output waves
    const int64_t o_stride = (int64_t)p.h_v * D;
    // outputs go to o, except the transition's (w, from token seg_start on)
    T* og = (role == 2 ? sp.w : reinterpret_cast<T*>(p.o)) + (int64_t)h * D + blk * L::cols + SW * cw + 4 * g4;
    const int64_t otok = role == 2 ? seg_start : 0;
    // O^T tile (ct, nt): rows 4g+i = columns SW cw + 16 ct + 4g + i, column
    // l16 = token pidx(th NTO + nt, l16) of the chunk
    f32x4 o[CT][NTO];
    int64_t orow[NTO];  // element offset of this lane's token row in each tile
#pragma unroll
    for (int nt = 0; nt < NTO; ++nt) orow[nt] = (int64_t)pidx<NT>(th * NTO + nt, l16) * o_stride;
    auto store_o = [&](int64_t t0, int Lc) {
      T* oc = og + (t0 - otok) * o_stride;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int nt = 0; nt < NTO; ++nt) {
          if (pidx<NT>(th * NTO + nt, l16) < Lc)
            *reinterpret_cast<uint2*>(oc + orow[nt] + 16 * ct) =
                make_uint2(pack_bf16x2(o[ct][nt][0], o[ct][nt][1]), pack_bf16x2(o[ct][nt][2], o[ct][nt][3]));
        }
    };
    __syncthreads();  // chunk 0 has landed; the initial state is published

    auto step = [&](int c, const unsigned char* cur, unsigned char* nxt) {
      if (c > 0) store_o(chunk_t0(c - 1), C);
      if constexpr (NM == 0) issue_next(c, nxt);
      const unsigned char* Q_t = cur + L::oQ;
      const unsigned char* P_t = cur + L::oP;
      const float* vec = reinterpret_cast<const float*>(cur + L::oVec);
      // Y^T = S Q^T, columns scaled by scale gamma rq
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int nt = 0; nt < NTO; ++nt) o[ct][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < D / 32; ++s) {
        frag as[CT], bq[NTO];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) as[ct] = frag_row_s<T, SS>(sS, colof(ct), 32 * s + 8 * g4, false);
#pragma unroll
        for (int nt = 0; nt < NTO; ++nt)
          bq[nt] = frag_row_s<T, SK>(Q_t, pidx<NT>(th * NTO + nt, l16), 32 * s + 8 * g4, false);
#pragma unroll
        for (int nt = 0; nt < NTO; ++nt)
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) M::mma(o[ct][nt], as[ct], bq[nt], false);
      }
#pragma unroll
      for (int nt = 0; nt < NTO; ++nt) {
        const float sc = vec[C + pidx<NT>(th * NTO + nt, l16)];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) o[ct][nt] *= sc;
      }
      barrier_vm<63>();  // B1
      // O^T += U^T P^T
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        frag au[CT], bp[NTO];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) au[ct] = frag_row_s<T, SU>(sU, colof(ct), HALF ? 4 * g4 : 32 * s + 8 * g4, HALF);
#pragma unroll
        for (int nt = 0; nt < NTO; ++nt)
          bp[nt] = frag_row_s<T, SC>(P_t, pidx<NT>(th * NTO + nt, l16), HALF ? 4 * g4 : 32 * s + 8 * g4, HALF);
#pragma unroll
        for (int nt = 0; nt < NTO; ++nt)
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) M::mma(o[ct][nt], au[ct], bp[nt], HALF);
      }
      __syncthreads();  // B2: the next chunk has landed
    };
    for (int c = 0; c < nch; c += 2) {
      step(c, sb0, sb1);
      if (c + 1 < nch) step(c + 1, sb1, sb0);
    }
    if (nch > 0) store_o(chunk_t0(nch - 1), chunk_len(nch - 1));
  } else {
    // ---------------------------------------------------------- mover waves
    // per chunk: the next chunk's loads, then the touches, which stay in
    // flight across B2 (only the loads before them are waited for)
    __syncthreads();  // chunk 0 has landed; the initial state is published
    for (int c = 0; c < nch; ++c) {
      issue_next(c, (c & 1) ? sb0 : sb1);
      __builtin_amdgcn_sched_barrier(0);
      if (touches) touch(c);
      barrier_vm<63>();      // B1 (nothing to wait for)
      barrier_vm<NTOUCH>();  // B2: this wave's loads of the next chunk have landed
    }
#pragma unroll
    for (int i = 0; i < NTOUCH; ++i) asm volatile("" ::"v"(tv[i]));
  }
}

// Every launched variant is instantiated explicitly: clang does not always
// emit the host launch stub of an implicitly instantiated kernel template
// whose body holds capturing lambdas.
#ifndef GDN_SCAN2_CT
#define GDN_SCAN2_CT 1
#endif
constexpr int kScan2Tiles = GDN_SCAN2_CT;  // 16-column tiles per wave
// output waves per column slice (each forms half of the chunk's tokens);
// one when the chunk has a single 16-token tile
#ifndef GDN_SCAN2_OS
#define GDN_SCAN2_OS 2
#endif
template <int C>
constexpr int kOutSplit = C >= 32 ? GDN_SCAN2_OS : 1;
// mover waves of the 32-column workgroups (the 64-column ones have no VGPR
// room for more waves: their output waves move the data)
#ifndef GDN_SCAN2_MOVERS
#define GDN_SCAN2_MOVERS 2
#endif
// (the layout needs two output waves per column slice: chunks of 32 tokens
// or more)
template <int C>
constexpr int kMovers = kOutSplit<C> == 2 ? GDN_SCAN2_MOVERS : 0;
// Two workgroup widths: 64 columns (four waves per role, two waves per SIMD)
// for launches that fill the chip, 32 columns (two waves per role) to spread
// a few long chains over twice as many CUs.
#define GDN_SCAN2(D, C) \
  template __global__ void scan2_kernel<D, C, kScan2Tiles, 4 / kScan2Tiles, kOutSplit<C>, 0>( \
      PrefillParams, const unsigned char*, ScanSplit); \
  template __global__ void scan2_kernel<D, C, kScan2Tiles, 2 / kScan2Tiles, kOutSplit<C>, kMovers<C>>( \
      PrefillParams, const unsigned char*, ScanSplit);
GDN_SCAN2(64, 16) GDN_SCAN2(64, 32) GDN_SCAN2(64, 64) GDN_SCAN2(128, 16) GDN_SCAN2(128, 32) GDN_SCAN2(128, 64)
#undef GDN_SCAN2

// ------------------------------------------------------------------ join
// After a split scan, on the second segment: o_t += S_m w_t, as
// O^T[j][t] = sum_i S_m[j][i] w[t][i] on MFMA (bf16 operands, fp32 sums; o
// is read and rounded once more), and the final state S_m Phi + S0 in fp32.
// Blocks [0, nstate): with a final state, h_v D/16 blocks of 16 state rows
// each (fp32 MFMA), first so that they overlap the rest.  Then blocks of
// kJoinTok tokens of V head h = block % h_v (a head's blocks share an XCD,
// and its S_m that L2): S_m (the bf16 copy the first segment wrote) and the
// w rows go to LDS through
// coalesced 16-byte loads, issued with the o rows they correct before any
// is used; wave w forms tokens [32 w, 32 w + 32) for every j, and the
// correction returns through LDS (fp32) so that o is read and written as
// whole 16-byte row pieces.
constexpr int kJoinTok = 128;
template <int D>
struct JoinLayout {
  static constexpr int RB = D * 2;  // bf16 rows of S_m and w
  static constexpr int oA = 0, oB = D * RB;
  static constexpr int in_bytes = oB + kJoinTok * RB;
  static constexpr int out_bytes = kJoinTok * D * 4;  // fp32 correction [t][j]
  static constexpr int bytes = in_bytes > out_bytes ? in_bytes : out_bytes;
};
template <int D>
__global__ __launch_bounds__(256) void join_kernel(PrefillParams p, ScanSplit sp, int64_t t_b, int nstate) {
  using M = Mma<__bf16>;
  using L = JoinLayout<D>;
  using SW = Swz<L::RB>;
  __shared__ __align__(16) unsigned char sm[L::bytes];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g4 = lane >> 4, l16 = lane & 15;
  const int64_t o_stride = (int64_t)p.h_v * D;
  const int64_t ntok = p.total_tokens - t_b;
  if ((int)blockIdx.x < nstate) {
    // final state rows 16 jb .. 16 jb + 15 of head h on fp32 MFMA: wave w
    // forms the 16x16 tiles nb = NPW w .. of S_m Phi + S0 as sums over kb of
    // (S_m block (jb, kb)) (Phi block (kb, nb)), every operand load issued
    // before the products
    constexpr int NB = D / 16, NPW = (NB + 3) / 4;
    const int h = blockIdx.x / NB, jb = blockIdx.x % NB;
    const size_t hs = (size_t)h * D * D;
    // the caller's final state: slot of the one sequence
    const size_t fs = ((size_t)(p.state_idx ? as_const(p.state_idx)[0] : 0) * p.h_v + h) * D * D;
    // y[kb]: the transposed S_m block in the accumulator layout, lane (g, c)
    // holding S_m[16 jb + c][16 kb + 4 g + i]
    f32x4 y[NB];
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
      const float4 v = *reinterpret_cast<const float4*>(sp.s_mid + hs + (size_t)(16 * jb + l16) * D + 16 * kb + 4 * g4);
      y[kb] = f32x4{v.x, v.y, v.z, v.w};
    }
#pragma unroll
    for (int t = 0; t < NPW; ++t) {
      const int nb = wave * NPW + t;
      if (nb >= NB) break;
      // lane (g, c): element (4 g + i, c) of block (., nb)
      auto at = [&](const float* m, int rb, int i) { return m + hs + (size_t)(16 * rb + 4 * g4 + i) * D + 16 * nb + l16; };
      f32x4 acc, w[NB];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = *at(sp.s_zero, jb, i);
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) w[kb][i] = *at(sp.phi, kb, i);
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) acc = mfma_tn(y[kb], w[kb], acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const size_t e = fs + (size_t)(16 * jb + 4 * g4 + i) * D + 16 * nb + l16;
        if (p.state_bf16) reinterpret_cast<__bf16*>(p.final_state)[e] = (__bf16)acc[i];
        else reinterpret_cast<float*>(p.final_state)[e] = acc[i];
      }
    }
    return;
  }
  const int bo = blockIdx.x - nstate;
  const int h = bo % p.h_v;
  const int64_t tb0 = (int64_t)(bo / p.h_v) * kJoinTok;  // relative to t_b
  // ---- loads: S_m (bf16), w and o rows (D/8 16-byte pieces per row);
  // rows past the segment re-read its last token
  constexpr int NSQ = D * D / 8 / 256, NWQ = kJoinTok * D / 8 / 256;
  const uint4* Sm = reinterpret_cast<const uint4*>(sp.s_mid_bf + (size_t)h * D * D);
  uint4 sv[NSQ];
  uint4 wv[NWQ], ov[NWQ];
#pragma unroll
  for (int q = 0; q < NSQ; ++q) sv[q] = Sm[tid + 256 * q];
#pragma unroll
  for (int q = 0; q < NWQ; ++q) {
    const int e = tid + 256 * q, t = e / (D / 8), pc = e % (D / 8);
    const int64_t tt = min(tb0 + t, ntok - 1);
    wv[q] = *reinterpret_cast<const uint4*>(sp.w + tt * o_stride + (int64_t)h * D + 8 * pc);
    ov[q] = *reinterpret_cast<const uint4*>(reinterpret_cast<const __bf16*>(p.o) + (t_b + tt) * o_stride +
                                            (int64_t)h * D + 8 * pc);
  }
#pragma unroll
  for (int q = 0; q < NSQ; ++q) {
    const int e = tid + 256 * q, j = e / (D / 8), c8 = e % (D / 8);
    *reinterpret_cast<uint4*>(sm + L::oA + SW::off(j, 16 * c8)) = sv[q];
  }
#pragma unroll
  for (int q = 0; q < NWQ; ++q) {
    const int e = tid + 256 * q, t = e / (D / 8), pc = e % (D / 8);
    *reinterpret_cast<uint4*>(sm + L::oB + SW::off(t, 16 * pc)) = wv[q];
  }
  __syncthreads();
  // ---- O^T tiles (jt, tt): rows j = 16 jt + 4g + i, column t = 32 wave + 16 tt + l16
  constexpr int JTN = D / 16, KS = D / 32;
  f32x4 acc[JTN][2];
#pragma unroll
  for (int jt = 0; jt < JTN; ++jt) acc[jt][0] = acc[jt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    typename M::frag bw[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
      bw[tt] = frag_row_s<__bf16, SW>(sm + L::oB, 32 * wave + 16 * tt + l16, 32 * s + 8 * g4, false);
#pragma unroll
    for (int jt = 0; jt < JTN; ++jt) {
      const typename M::frag a = frag_row_s<__bf16, SW>(sm + L::oA, 16 * jt + l16, 32 * s + 8 * g4, false);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) M::mma(acc[jt][tt], a, bw[tt], false);
    }
  }
  __syncthreads();  // S_m and w are dead: the bytes take the fp32 correction
  // [t][j] fp32, float4 column slots xor-swizzled by t so that the 16 lanes
  // of a group (16 tokens, one j slot) write 16 different bank groups
  auto cor = [&](int t, int j4) -> float4* {
    return reinterpret_cast<float4*>(sm) + t * (D / 4) + (j4 ^ (t % (D / 4)));
  };
#pragma unroll
  for (int jt = 0; jt < JTN; ++jt)
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
      *cor(32 * wave + 16 * tt + l16, 4 * jt + g4) = make_float4(acc[jt][tt][0], acc[jt][tt][1], acc[jt][tt][2], acc[jt][tt][3]);
  __syncthreads();
#pragma unroll
  for (int q = 0; q < NWQ; ++q) {
    const int e = tid + 256 * q, t = e / (D / 8), pc = e % (D / 8);
    if (tb0 + t >= ntok) continue;
    const float4 c0 = *cor(t, 2 * pc), c1 = *cor(t, 2 * pc + 1);
    const uint4 o = ov[q];
    const uint4 r = make_uint4(pack_bf16x2(bf16_lo(o.x) + c0.x, bf16_hi(o.x) + c0.y),
                               pack_bf16x2(bf16_lo(o.y) + c0.z, bf16_hi(o.y) + c0.w),
                               pack_bf16x2(bf16_lo(o.z) + c1.x, bf16_hi(o.z) + c1.y),
                               pack_bf16x2(bf16_lo(o.w) + c1.z, bf16_hi(o.w) + c1.w));
    *reinterpret_cast<uint4*>(reinterpret_cast<__bf16*>(p.o) + (t_b + tb0 + t) * o_stride + (int64_t)h * D + 8 * pc) = r;
  }
}

// ------------------------------------------------------------- fused scan
// bf16 at chunk 32 or 64: one launch runs the whole chunked recurrence with
// each chunk's preparation folded in, so the call reads q, k, v, g and beta
// once and writes o and the states, and nothing in between leaves the CU.
// One workgroup per (sequence, V head, block of 16 NC CT d_v columns).  Per
// chunk c there are two barriers, B1 and B2; between them:
//   phase 1  chain waves (NC, 16 CT columns each): X1 = K S^T, R, U = Tb R;
//              U is published (bf16); S^T <- gamma_last S^T + K^T diag(e rk)
//              U in registers;
//            output waves (NC, 16 CT columns each): Y = Q S^T (raw q rows)
//              with the squared row
//              norms of q from the same fragments, then the diagonal 16x16
//              tiles of chunk c+1's Q K^T with their decay masks (into P);
//            prep wave 0: the diagonal tiles of chunk c+1's K K^T, the row
//              norms of k from their diagonals, and the inverses of the
//              diagonal blocks of I + A by forward substitution in registers
//              (one lane per column, the other columns' entries broadcast
//              across the lanes of a row);
//            prep waves 1-3: the tiles of chunk c+1's K K^T and Q K^T below
//              the diagonal blocks with their decay masks only (one mask
//              serves both): the row and column scalings come later;
//   phase 2  chain: the new S published;
//            output: O = scale rq (gamma Y + P diag(rk) U), stored;
//            prep waves: the blocks of T = (I + A)^-1 below the diagonal
//              blocks, split by column block (bf16 MFMA products, A's
//              scalings applied as its blocks are converted), written as
//              Tb = T diag(beta); the chunk's row scalars; then chunk c+2's
//              raw rows, loaded to registers during the previous chunk, into
//              the raw buffer chunk c has freed, with beta and the
//              cumulative log-decay; then chunk c+3's loads.
// With the norms folded in as row and column scalings, a partial chunk needs
// no zeroing: rows past its end repeat its last row, and beta = g = 0 there
// makes their rows of A, Tb and U zero.  The blocks of Tb and P above the
// diagonal blocks stay zero and are cleared once.
// Two raw buffers (K, Q, the block's V columns, per-token scalars) and two
// prep buffers (Tb, P, per-token scalars) alternate by chunk parity; the
// chunk loop is unrolled by two so that every LDS address is static.  A raw
// buffer is free after B1 of the chunk that used it: the chain holds its K^T
// fragments in registers by then and the outputs read Q in phase 1 only.
// A wave64 VALU instruction costs four cycles and an LDS round trip far
// more under load, so per-lane LDS offsets are computed once, outside the
// loop, and the preparation keeps its serial steps (the substitution, the
// prefix sum of g) in registers with cross-lane moves.

// a's upper 32 lanes and b's lower 32 lanes trade places
__device__ __forceinline__ void swap_hi32(float& a, float& b) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  const uint32_t x = s[0];
  const uint32_t y = s[1];
  a = __uint_as_float(x);
  b = __uint_as_float(y);
}
// a's odd rows of 16 lanes and b's even rows trade places
__device__ __forceinline__ void swap_odd16(float& a, float& b) {
  const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  const uint32_t x = s[0];
  const uint32_t y = s[1];
  a = __uint_as_float(x);
  b = __uint_as_float(y);
}
// inclusive prefix sum over the 64 lanes: shifts within rows of 16, then
// the totals of the rows below
__device__ __forceinline__ float wave_prefix_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xF, 0xF, true));  // row_shr:1
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xF, 0xF, true));  // row_shr:2
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xF, 0xF, true));  // row_shr:4
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xF, 0xF, true));  // row_shr:8
  const int row = (int)(threadIdx.x & 63) >> 4;
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 15));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 31));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 47));
  return x + (row >= 1 ? r0 : 0.f) + (row >= 2 ? r1 : 0.f) + (row >= 3 ? r2 : 0.f);
}
// Forward substitution for one column of the inverse of a unit lower
// triangular 16x16 block: lane j of a row of 16 holds column j of the
// negated strict lower part in nn; on return t (e_k on entry, k the lane's
// column) is column k of the inverse.  Step j adds column j times t[j] to
// the entries below j, column j reaching every lane of the row through a
// row broadcast (DPP row_newbcast:j) folded into the multiply-add.  Each
// step is one asm block opened by two wait states, which a VALU write of a
// register before a DPP read of it requires.
__device__ __forceinline__ void subst16(float (&t)[16], const float (&nn)[16]) {
  asm volatile("s_nop 1\n\tv_fmac_f32_dpp %0, %15, %30 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %1, %16, %30 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %2, %17, %30 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %3, %18, %30 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %4, %19, %30 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %5, %20, %30 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %6, %21, %30 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %7, %22, %30 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %8, %23, %30 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %9, %24, %30 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %10, %25, %30 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %11, %26, %30 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %12, %27, %30 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %13, %28, %30 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %14, %29, %30 row_newbcast:0 row_mask:0xf bank_mask:0xf"
               : "+v"(t[1]), "+v"(t[2]), "+v"(t[3]), "+v"(t[4]), "+v"(t[5]), "+v"(t[6]), "+v"(t[7]), "+v"(t[8]), "+v"(t[9]), "+v"(t[10]), "+v"(t[11]), "+v"(t[12]), "+v"(t[13]), "+v"(t[14]), "+v"(t[15])
               : "v"(nn[1]), "v"(nn[2]), "v"(nn[3]), "v"(nn[4]), "v"(nn[5]), "v"(nn[6]), "v"(nn[7]), "v"(nn[8]), "v"(nn[9]), "v"(nn[10]), "v"(nn[11]), "v"(nn[12]), "v"(nn[13]), "v"(nn[14]), "v"(nn[15]), "v"(t[0]));
  asm volatile("s_nop 1\n\tv_fmac_f32_dpp %0, %14, %28 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %1, %15, %28 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %2, %16, %28 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %3, %17, %28 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %4, %18, %28 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %5, %19, %28 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %6, %20, %28 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %7, %21, %28 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %8, %22, %28 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %9, %23, %28 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %10, %24, %28 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %11, %25, %28 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %12, %26, %28 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %13, %27, %28 row_newbcast:1 row_mask:0xf bank_mask:0xf"
               : "+v"(t[2]), "+v"(t[3]), "+v"(t[4]), "+v"(t[5]), "+v"(t[6]), "+v"(t[7]), "+v"(t[8]), "+v"(t[9]), "+v"(t[10]), "+v"(t[11]), "+v"(t[12]), "+v"(t[13]), "+v"(t[14]), "+v"(t[15])
               : "v"(nn[2]), "v"(nn[3]), "v"(nn[4]), "v"(nn[5]), "v"(nn[6]), "v"(nn[7]), "v"(nn[8]), "v"(nn[9]), "v"(nn[10]), "v"(nn[11]), "v"(nn[12]), "v"(nn[13]), "v"(nn[14]), "v"(nn[15]), "v"(t[1]));
  asm volatile("s_nop 1\n\tv_fmac_f32_dpp %0, %13, %26 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %1, %14, %26 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %2, %15, %26 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %3, %16, %26 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %4, %17, %26 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %5, %18, %26 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %6, %19, %26 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %7, %20, %26 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %8, %21, %26 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %9, %22, %26 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %10, %23, %26 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %11, %24, %26 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %12, %25, %26 row_newbcast:2 row_mask:0xf bank_mask:0xf"
               : "+v"(t[3]), "+v"(t[4]), "+v"(t[5]), "+v"(t[6]), "+v"(t[7]), "+v"(t[8]), "+v"(t[9]), "+v"(t[10]), "+v"(t[11]), "+v"(t[12]), "+v"(t[13]), "+v"(t[14]), "+v"(t[15])
               : "v"(nn[3]), "v"(nn[4]), "v"(nn[5]), "v"(nn[6]), "v"(nn[7]), "v"(nn[8]), "v"(nn[9]), "v"(nn[10]), "v"(nn[11]), "v"(nn[12]), "v"(nn[13]), "v"(nn[14]), "v"(nn[15]), "v"(t[2]));
  asm volatile("s_nop 1\n\tv_fmac_f32_dpp %0, %12, %24 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %1, %13, %24 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %2, %14, %24 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %3, %15, %24 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %4, %16, %24 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %5, %17, %24 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %6, %18, %24 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %7, %19, %24 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %8, %20, %24 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %9, %21, %24 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %10, %22, %24 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %11, %23, %24 row_newbcast:3 row_mask:0xf bank_mask:0xf"
               : "+v"(t[4]), "+v"(t[5]), "+v"(t[6]), "+v"(t[7]), "+v"(t[8]), "+v"(t[9]), "+v"(t[10]), "+v"(t[11]), "+v"(t[12]), "+v"(t[13]), "+v"(t[14]), "+v"(t[15])
               : "v"(nn[4]), "v"(nn[5]), "v"(nn[6]), "v"(nn[7]), "v"(nn[8]), "v"(nn[9]), "v"(nn[10]), "v"(nn[11]), "v"(nn[12]), "v"(nn[13]), "v"(nn[14]), "v"(nn[15]), "v"(t[3]));
  asm volatile("s_nop 1\n\tv_fmac_f32_dpp %0, %11, %22 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %1, %12, %22 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %2, %13, %22 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %3, %14, %22 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %4, %15, %22 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %5, %16, %22 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %6, %17, %22 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %7, %18, %22 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %8, %19, %22 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %9, %20, %22 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %10, %21, %22 row_newbcast:4 row_mask:0xf bank_mask:0xf"
               : "+v"(t[5]), "+v"(t[6]), "+v"(t[7]), "+v"(t[8]), "+v"(t[9]), "+v"(t[10]), "+v"(t[11]), "+v"(t[12]), "+v"(t[13]), "+v"(t[14]), "+v"(t[15])
               : "v"(nn[5]), "v"(nn[6]), "v"(nn[7]), "v"(nn[8]), "v"(nn[9]), "v"(nn[10]), "v"(nn[11]), "v"(nn[12]), "v"(nn[13]), "v"(nn[14]), "v"(nn[15]), "v"(t[4]));
  asm volatile("s_nop 1\n\tv_fmac_f32_dpp %0, %10, %20 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %1, %11, %20 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %2, %12, %20 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %3, %13, %20 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %4, %14, %20 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %5, %15, %20 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %6, %16, %20 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %7, %17, %20 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %8, %18, %20 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %9, %19, %20 row_newbcast:5 row_mask:0xf bank_mask:0xf"
               : "+v"(t[6]), "+v"(t[7]), "+v"(t[8]), "+v"(t[9]), "+v"(t[10]), "+v"(t[11]), "+v"(t[12]), "+v"(t[13]), "+v"(t[14]), "+v"(t[15])
               : "v"(nn[6]), "v"(nn[7]), "v"(nn[8]), "v"(nn[9]), "v"(nn[10]), "v"(nn[11]), "v"(nn[12]), "v"(nn[13]), "v"(nn[14]), "v"(nn[15]), "v"(t[5]));
  asm volatile("s_nop 1\n\tv_fmac_f32_dpp %0, %9, %18 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %1, %10, %18 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %2, %11, %18 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %3, %12, %18 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %4, %13, %18 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %5, %14, %18 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %6, %15, %18 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %7, %16, %18 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %8, %17, %18 row_newbcast:6 row_mask:0xf bank_mask:0xf"
               : "+v"(t[7]), "+v"(t[8]), "+v"(t[9]), "+v"(t[10]), "+v"(t[11]), "+v"(t[12]), "+v"(t[13]), "+v"(t[14]), "+v"(t[15])
               : "v"(nn[7]), "v"(nn[8]), "v"(nn[9]), "v"(nn[10]), "v"(nn[11]), "v"(nn[12]), "v"(nn[13]), "v"(nn[14]), "v"(nn[15]), "v"(t[6]));
  asm volatile("s_nop 1\n\tv_fmac_f32_dpp %0, %8, %16 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %1, %9, %16 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %2, %10, %16 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %3, %11, %16 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %4, %12, %16 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %5, %13, %16 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %6, %14, %16 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %7, %15, %16 row_newbcast:7 row_mask:0xf bank_mask:0xf"
               : "+v"(t[8]), "+v"(t[9]), "+v"(t[10]), "+v"(t[11]), "+v"(t[12]), "+v"(t[13]), "+v"(t[14]), "+v"(t[15])
               : "v"(nn[8]), "v"(nn[9]), "v"(nn[10]), "v"(nn[11]), "v"(nn[12]), "v"(nn[13]), "v"(nn[14]), "v"(nn[15]), "v"(t[7]));
  asm volatile("s_nop 1\n\tv_fmac_f32_dpp %0, %7, %14 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %1, %8, %14 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %2, %9, %14 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %3, %10, %14 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %4, %11, %14 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %5, %12, %14 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %6, %13, %14 row_newbcast:8 row_mask:0xf bank_mask:0xf"
               : "+v"(t[9]), "+v"(t[10]), "+v"(t[11]), "+v"(t[12]), "+v"(t[13]), "+v"(t[14]), "+v"(t[15])
               : "v"(nn[9]), "v"(nn[10]), "v"(nn[11]), "v"(nn[12]), "v"(nn[13]), "v"(nn[14]), "v"(nn[15]), "v"(t[8]));
  asm volatile("s_nop 1\n\tv_fmac_f32_dpp %0, %6, %12 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %1, %7, %12 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %2, %8, %12 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %3, %9, %12 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %4, %10, %12 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %5, %11, %12 row_newbcast:9 row_mask:0xf bank_mask:0xf"
               : "+v"(t[10]), "+v"(t[11]), "+v"(t[12]), "+v"(t[13]), "+v"(t[14]), "+v"(t[15])
               : "v"(nn[10]), "v"(nn[11]), "v"(nn[12]), "v"(nn[13]), "v"(nn[14]), "v"(nn[15]), "v"(t[9]));
  asm volatile("s_nop 1\n\tv_fmac_f32_dpp %0, %5, %10 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %1, %6, %10 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %2, %7, %10 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %3, %8, %10 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %4, %9, %10 row_newbcast:10 row_mask:0xf bank_mask:0xf"
               : "+v"(t[11]), "+v"(t[12]), "+v"(t[13]), "+v"(t[14]), "+v"(t[15])
               : "v"(nn[11]), "v"(nn[12]), "v"(nn[13]), "v"(nn[14]), "v"(nn[15]), "v"(t[10]));
  asm volatile("s_nop 1\n\tv_fmac_f32_dpp %0, %4, %8 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %1, %5, %8 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %2, %6, %8 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %3, %7, %8 row_newbcast:11 row_mask:0xf bank_mask:0xf"
               : "+v"(t[12]), "+v"(t[13]), "+v"(t[14]), "+v"(t[15])
               : "v"(nn[12]), "v"(nn[13]), "v"(nn[14]), "v"(nn[15]), "v"(t[11]));
  asm volatile("s_nop 1\n\tv_fmac_f32_dpp %0, %3, %6 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %1, %4, %6 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %2, %5, %6 row_newbcast:12 row_mask:0xf bank_mask:0xf"
               : "+v"(t[13]), "+v"(t[14]), "+v"(t[15])
               : "v"(nn[13]), "v"(nn[14]), "v"(nn[15]), "v"(t[12]));
  asm volatile("s_nop 1\n\tv_fmac_f32_dpp %0, %2, %4 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\tv_fmac_f32_dpp %1, %3, %4 row_newbcast:13 row_mask:0xf bank_mask:0xf"
               : "+v"(t[14]), "+v"(t[15])
               : "v"(nn[14]), "v"(nn[15]), "v"(t[13]));
  asm volatile("s_nop 1\n\tv_fmac_f32_dpp %0, %1, %2 row_newbcast:14 row_mask:0xf bank_mask:0xf"
               : "+v"(t[15])
               : "v"(nn[15]), "v"(t[14]));
}

// r[e] = x of lane 4Q + e of the lane's row of 16 (DPP row_newbcast)
template <int Q>
__device__ __forceinline__ void row_bcast4(float (&r)[4], float x) {
  asm volatile("s_nop 1\n\t"
               "v_mov_b32_dpp %0, %4 row_newbcast:%c5 row_mask:0xf bank_mask:0xf\n\t"
               "v_mov_b32_dpp %1, %4 row_newbcast:%c6 row_mask:0xf bank_mask:0xf\n\t"
               "v_mov_b32_dpp %2, %4 row_newbcast:%c7 row_mask:0xf bank_mask:0xf\n\t"
               "v_mov_b32_dpp %3, %4 row_newbcast:%c8 row_mask:0xf bank_mask:0xf"
               : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
               : "v"(x), "i"(4 * Q), "i"(4 * Q + 1), "i"(4 * Q + 2), "i"(4 * Q + 3));
}

template <int D, int C, int NC, int CT, bool W>
struct FusedLayout {
  static constexpr int NT = C / 16, DT = D / 16;
  static constexpr int cols = 16 * NC * CT;
  static_assert(!W || (cols == D && CT == 2), "a wide workgroup holds every d_v column, 32 per chain wave");
  static constexpr int RBK = D * 2, RBC = C * 2, RBV = cols * 2, RBS = D * 2, RBU = C * 2;
  using SK = Swz<RBK>;
  using SC = Swz<RBC>;
  using SV = SwzT<RBV, RowV<NT, RBV / 16>>;
  using SS = SwzT<RBS, RowSeq<RBS>>;
  using SU = SwzT<RBU, RowSeq<RBU>>;
  // raw buffer: K, Q rows [C][D] (swizzled), V [C][cols], then per-token
  // fp32 rows: beta, G log2(e) (cumulative log-decay in base 2), rk
  static constexpr int rK = 0, rQ = C * RBK, rV = 2 * C * RBK, rSc = rV + C * RBV;
  static constexpr int raw = rSc + 12 * C;
  // prep buffer: Tb, P~ [C][C] (swizzled), then per-token fp32 rows:
  // gamma rk (0 without the erase), gamma, e rk, gamma_last, rk, and (wide
  // workgroups) scale rq
  static constexpr int NVEC = 6;
  static constexpr int pTb = 0, pP = C * RBC, pVec = 2 * C * RBC;
  static constexpr int prep = pVec + 4 * NVEC * C;
  static constexpr int LDF = C + 4;  // fp32 A / T rows
  // the published state and U: only where separate output waves read them
  static constexpr int sbytes = W ? 16 : cols * RBS, ubytes = W ? 16 : cols * RBU;
  static constexpr int bytes = 2 * raw + 2 * prep + C * LDF * 4 + sbytes + ubytes;
  static constexpr int threads = 64 * (W ? NC + 4 : 2 * NC + 4);
  static_assert(NT == 2 || NT == 4, "chunks of 32 or 64 tokens");
};

constexpr float kLog2e = 1.4426950408889634f;


// Off-diagonal tile pairs (row block mt > column block tj) of prep wave pw
// (1..3), chosen so that a wave's pairs share operand tiles
struct TilePair { int mt, tj; };
template <int NT>
constexpr int pairs_of(int pw) { return NT == 2 ? (pw == 1 ? 1 : 0) : 2; }
template <int NT>
constexpr TilePair pair_at(int pw, int i) {
  return NT == 2 ? TilePair{1, 0}
       : pw == 1 ? (i == 0 ? TilePair{1, 0} : TilePair{2, 0})
       : pw == 2 ? (i == 0 ? TilePair{3, 0} : TilePair{3, 1})
                 : (i == 0 ? TilePair{2, 1} : TilePair{3, 2});
}
template <int D, int C, int NC, int CT, bool W>
__global__ __launch_bounds__(64 * (W ? NC + 4 : 2 * NC + 4)) void fused_kernel(PrefillParams p, const unsigned char* ws) {
  using L = FusedLayout<D, C, NC, CT, W>;
  using T = __bf16;
  using M = Mma<T>;
  using frag = typename M::frag;
  using SK = typename L::SK;
  using SC = typename L::SC;
  using SV = typename L::SV;
  using SS = typename L::SS;
  using SU = typename L::SU;
  constexpr int NT = L::NT, DT = L::DT, DKS = D / 32, KS = NT / 2, LDF = L::LDF;
  constexpr int NB = D / L::cols;
  __shared__ __align__(16) unsigned char raw0[L::raw];
  __shared__ __align__(16) unsigned char raw1[L::raw];
  __shared__ __align__(16) unsigned char prp0[L::prep];
  __shared__ __align__(16) unsigned char prp1[L::prep];
  __shared__ __align__(16) float sA[C * LDF];
  __shared__ __align__(16) unsigned char sS[L::sbytes];
  __shared__ __align__(16) unsigned char sU[L::ubytes];

  const PlanView plan = plan_view(p, ws, C);
  const ScanSlot slot = scan_slot(p, plan, NB);
  if (!slot.valid) return;
  const int blk = slot.blk, h = slot.h, n = slot.n;
  const int hq = h / (p.h_v / p.h_qk);
  // the wave index is uniform across a wave: keep it (and every role and job
  // parameter derived from it) in scalar registers
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4, l16 = lane & 15;
  const int64_t seq_start = p.cu_seqlens ? as_const(p.cu_seqlens)[n] : 0;
  const int64_t seq_end = p.cu_seqlens ? as_const(p.cu_seqlens)[n + 1] : p.total_tokens;
  const int nch = plan.off(n + 1) - plan.off(n);
  auto chunk_t0 = [&](int c) __attribute__((always_inline)) { return seq_start + (int64_t)c * C; };
  auto chunk_len = [&](int c) __attribute__((always_inline)) { return (int)min((int64_t)C, seq_end - chunk_t0(c)); };

  // roles: waves w and w + 4 share a SIMD.  Chain waves come first (one per
  // SIMD), then the output waves, then the four prep waves, numbered so
  // that prep wave 0 (the diagonal solve) sits beside an output wave rather
  // than a chain wave when the layout allows it.  A wide workgroup has no
  // output waves: its chain waves form the outputs of their own columns,
  // and with two chain waves prep waves 0 and 1 have a SIMD each.
  const bool chain = wave < NC;
  const bool outw = !W && wave >= NC && wave < 2 * NC;
  const bool prepw = wave >= (W ? NC : 2 * NC);
  const int pi = !prepw ? -1 : W ? wave - NC : (wave - 2 * NC + (NC == 2 ? 2 : 0)) & 3;
  const int lt = prepw ? pi * 64 + lane : 0;  // loader thread 0..255

  // fragment reads of the K, Q tiles (token rows 16 t + l16, d_k 32 s + 8 g
  // .. + 7): byte offsets inside a tile, computed once
  uint32_t fo[NT][DKS];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int s = 0; s < DKS; ++s) fo[t][s] = (uint32_t)SK::off(t * 16 + l16, (32 * s + 8 * g4) * 2);
  auto kfrag = [&](const unsigned char* tile, int t, int s) __attribute__((always_inline)) {
    return __builtin_bit_cast(frag, *reinterpret_cast<const uint4*>(tile + fo[t][s]));
  };

  // ---------------------------------------------------------- decay masks
  // Gram tiles are formed transposed: tile (mt, tj) holds rows j = 16 tj +
  // 4g + i, column r = 16 mt + l16 of K K^T (or K Q^T), so that a lane holds
  // row r, columns j0 .. j0 + 3 of A (or P).  With raw rows k, q:
  //   A_rj = beta_r rk_r e^{G_r - G_j} rk_j (k_r . k_j)         (j <  r)
  //   P_rj = scale rq_r e^{G_r - G_j} rk_j (q_r . k_j)          (j <= r)
  // The masks write only e^{G_r - G_j} times the raw product (A~, P~); the
  // scalars hold G log2(e), so e^{G_r - G_j} = 2^{G2_r - G2_j} <= 1.
  auto gram = [&](const unsigned char* A_t, const unsigned char* B_t, int mt, int tj) __attribute__((always_inline)) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < DKS; ++s) M::mma(acc, kfrag(A_t, tj, s), kfrag(B_t, mt, s), false);
    return acc;
  };
  // decay of a lane's four entries (0 where the mask removes them: j > r,
  // or j >= r when strict)
  // (lx, gx: the lane's l16 and g4, passed where they are formed afresh)
  auto decay_l = [&](const float* sc, int mt, int tj, bool strict, float (&w)[4], int lx, int gx) __attribute__((always_inline)) {
    const int r = mt * 16 + lx, j0 = tj * 16 + 4 * gx;
    const float Gr = sc[C + r];
    const float4 Gj = *reinterpret_cast<const float4*>(sc + C + j0);
    const float gj[4] = {Gj.x, Gj.y, Gj.z, Gj.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x = __builtin_amdgcn_exp2f(Gr - gj[i]);
      w[i] = mt > tj ? x : (strict ? (j0 + i < r ? x : 0.f) : (j0 + i <= r ? x : 0.f));
    }
  };
  auto decay = [&](const float* sc, int mt, int tj, bool strict, float (&w)[4]) __attribute__((always_inline)) {
    decay_l(sc, mt, tj, strict, w, l16, g4);
  };
  auto put_p_l = [&](unsigned char* P_s, int mt, int tj, const float (&w)[4], const f32x4& qk, int lx, int gx) __attribute__((always_inline)) {
    const int r = mt * 16 + lx, j0 = tj * 16 + 4 * gx;
    *reinterpret_cast<uint2*>(P_s + SC::off(r, j0 * 2)) =
        make_uint2(pack_bf16x2(w[0] * qk[0], w[1] * qk[1]), pack_bf16x2(w[2] * qk[2], w[3] * qk[3]));
  };
  auto put_p = [&](unsigned char* P_s, int mt, int tj, const float (&w)[4], const f32x4& qk) __attribute__((always_inline)) {
    put_p_l(P_s, mt, tj, w, qk, l16, g4);
  };

  // ------------------------------------------------- raw rows (prep waves)
  constexpr int NLD = 256;
  constexpr int RT = D / 8;                      // 16-byte pieces per K / Q row
  constexpr int NKP = (C * RT + NLD - 1) / NLD;  // K (and Q) pieces per loader thread
  constexpr int VT = L::cols / 8;                // pieces per row of this block's V
  constexpr int NVP = (C * VT + NLD - 1) / NLD;
  gdn_u4 kr[NKP], qr[NKP], vr[NVP];  // native vectors: kept in registers
  float gr = 0.f, br = 0.f;
  // per piece: global offsets inside a full chunk (bytes from the chunk's
  // first row) and LDS offsets in the tile, computed once
  uint32_t kgo[NKP], qgo[NKP], kso[NKP], vgo[NVP], vso[NVP];
#pragma unroll
  for (int i = 0; i < NKP; ++i) {
    const int e = min(lt + NLD * i, C * RT - 1);
    const int r = e / RT, c0 = (e % RT) * 8;
    kgo[i] = (uint32_t)(r * p.k_stride + c0) * 2u;
    qgo[i] = (uint32_t)(r * p.q_stride + c0) * 2u;
    kso[i] = (uint32_t)SK::off(r, c0 * 2);
  }
#pragma unroll
  for (int i = 0; i < NVP; ++i) {
    const int e = min(lt + NLD * i, C * VT - 1);
    const int r = e / VT, c0 = (e % VT) * 8;
    vgo[i] = (uint32_t)(r * p.v_stride + c0) * 2u;
    vso[i] = (uint32_t)SV::off(r, c0 * 2);
  }
  const unsigned char* kg = reinterpret_cast<const unsigned char*>(reinterpret_cast<const T*>(p.k) + (int64_t)hq * D);
  const unsigned char* qg = reinterpret_cast<const unsigned char*>(reinterpret_cast<const T*>(p.q) + (int64_t)hq * D);
  const unsigned char* vg =
      reinterpret_cast<const unsigned char*>(reinterpret_cast<const T*>(p.v) + (int64_t)h * D + blk * L::cols);
  // chunk c's rows into registers; in a partial chunk, rows past its end
  // re-read its last row
  auto load_raw = [&](int c) __attribute__((always_inline)) {
    const int64_t t0 = chunk_t0(c);
    const int Lc = chunk_len(c);
    const unsigned char* kc = kg + t0 * p.k_stride * 2;
    const unsigned char* qc = qg + t0 * p.q_stride * 2;
    const unsigned char* vc = vg + t0 * p.v_stride * 2;
    if (Lc == C) {
#pragma unroll
      for (int i = 0; i < NKP; ++i) {
        kr[i] = *reinterpret_cast<const gdn_u4*>(kc + kgo[i]);
        qr[i] = *reinterpret_cast<const gdn_u4*>(qc + qgo[i]);
      }
#pragma unroll
      for (int i = 0; i < NVP; ++i) vr[i] = *reinterpret_cast<const gdn_u4*>(vc + vgo[i]);
    } else {
#pragma unroll
      for (int i = 0; i < NKP; ++i) {
        const int e = min(lt + NLD * i, C * RT - 1);
        const int64_t r = min(e / RT, Lc - 1);
        const int c0 = (e % RT) * 8;
        kr[i] = *reinterpret_cast<const gdn_u4*>(kc + (r * p.k_stride + c0) * 2);
        qr[i] = *reinterpret_cast<const gdn_u4*>(qc + (r * p.q_stride + c0) * 2);
      }
#pragma unroll
      for (int i = 0; i < NVP; ++i) {
        const int e = min(lt + NLD * i, C * VT - 1);
        const int64_t r = min(e / VT, Lc - 1);
        vr[i] = *reinterpret_cast<const gdn_u4*>(vc + (r * p.v_stride + (e % VT) * 8) * 2);
      }
    }
    if (pi == 1) {
      const int64_t r = t0 + min(lane, Lc - 1);
      gr = p.g[r * p.h_v + h];
      br = p.beta[r * p.h_v + h];
    }
  };
  // beta and G log2(e) of chunk c into raw buffer b (G the cumulative sum of
  // g; beta = g = 0 past the chunk's end), from the registers of prep wave 1
  auto store_sc = [&](int c, unsigned char* b) __attribute__((always_inline)) {
    const int Lc = chunk_len(c);
    const float G = wave_prefix_sum(lane < Lc ? gr : 0.f);
    float* sc = reinterpret_cast<float*>(b + L::rSc);
    if (lane < C) {
      sc[lane] = lane < Lc ? br : 0.f;
      sc[C + lane] = G * kLog2e;
    }
  };
  // the registers of chunk c into raw buffer b, with the scalars.  Prep wave
  // 1 holds g and beta.
  auto store_raw = [&](int c, unsigned char* b) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NKP; ++i) {
      if (NLD * (i + 1) <= C * RT || lt + NLD * i < C * RT) {
        *reinterpret_cast<gdn_u4*>(b + L::rK + kso[i]) = kr[i];
        *reinterpret_cast<gdn_u4*>(b + L::rQ + kso[i]) = qr[i];
      }
    }
#pragma unroll
    for (int i = 0; i < NVP; ++i)
      if (NLD * (i + 1) <= C * VT || lt + NLD * i < C * VT) *reinterpret_cast<gdn_u4*>(b + L::rV + vso[i]) = vr[i];
    if (pi == 1) store_sc(c, b);
  };
  // Wide workgroups: the four prep waves copy a chunk's K, Q and V rows
  // straight into the raw buffer (16 bytes per lane; the lane fetches the
  // global piece whose swizzled slot is its LDS position), and prep wave 1
  // loads g and beta into registers.  A full chunk uses per-lane offsets
  // computed once; a partial one clamps rows past its end to its last row.
  DmaPlan<SK, C, 4> pk, pq;
  DmaPlan<SV, C, 4> pv;
  const int64_t vrow = p.v_stride * 2;
  const bool dfast = p.q_stride * 2 * C < (1ll << 31) && p.k_stride * 2 * C < (1ll << 31) && vrow * C < (1ll << 31);
  if (W && prepw && dfast) {
    pk.init((uint32_t)(p.k_stride * 2), pi, lane);
    pq.init((uint32_t)(p.q_stride * 2), pi, lane);
    pv.init((uint32_t)vrow, pi, lane);
  }
  auto dma_raw = [&](int c, unsigned char* b) __attribute__((always_inline)) {
    const int64_t t0 = chunk_t0(c);
    const int Lc = chunk_len(c);
    const unsigned char* kc = kg + t0 * p.k_stride * 2;
    const unsigned char* qc = qg + t0 * p.q_stride * 2;
    const unsigned char* vc = vg + t0 * vrow;
    if (dfast && Lc == C) {
      pk.issue(b + L::rK, kc, pi, lane);
      pq.issue(b + L::rQ, qc, pi, lane);
      pv.issue(b + L::rV, vc, pi, lane);
    } else {
      dma_tile_s<SK, C, 4>(b + L::rK, kc, p.k_stride * 2, Lc, pi, lane);
      dma_tile_s<SK, C, 4>(b + L::rQ, qc, p.q_stride * 2, Lc, pi, lane);
      dma_tile_s<SV, C, 4>(b + L::rV, vc, vrow, Lc, pi, lane);
    }
  };
  // L2 prefetch for wide workgroups: two 4-byte loads per loader slot lt
  // (0..255) touch every 128-byte line of a chunk's K, Q and V rows and its
  // g and beta entries, so that the direct-to-LDS copy after B1 reads L2
  // rather than HBM.  Prep waves 1-3 issue them at the start of phase 1,
  // while the load path is idle (wave 1 also takes wave 0's slots); both
  // loads are issued on every call (a chunk past the end touches the last
  // chunk again), and the next call waits for them before reusing their
  // registers, a step later.
  uint32_t tv0 = 0u, tv1 = 0u, tv2 = 0u, tv3 = 0u;
  auto touch_lt = [&](int c, int lx, uint32_t& va, uint32_t& vb) __attribute__((always_inline)) {
    asm volatile("" ::"v"(va), "v"(vb));
    const int cc = min(c, nch - 1);
    const int64_t t0 = chunk_t0(cc);
    const int Lc = chunk_len(cc);
    const int i = lx & 127, half = (i & 1) * 128 < D * 2 ? (i & 1) * 128 : 0;
    const int64_t r = t0 + min(i >> 1, Lc - 1);
    const unsigned char* a0 = lx < 128 ? kg + r * p.k_stride * 2 + half : qg + r * p.q_stride * 2 + half;
    const unsigned char* a1;
    if (lx < 128) {
      a1 = vg + r * vrow + half;
    } else {
      const int64_t rg = t0 + min(lx & 63, Lc - 1);
      a1 = reinterpret_cast<const unsigned char*>((lx < 192 ? p.g : p.beta) + rg * p.h_v + h);
    }
    va = *reinterpret_cast<const uint32_t*>(a0);
    vb = *reinterpret_cast<const uint32_t*>(a1);
  };
  auto touch = [&](int c) __attribute__((always_inline)) {  // prep waves 1-3
    touch_lt(c, lt, tv0, tv1);
    if (pi == 1) touch_lt(c, lane, tv2, tv3);
  };
  auto load_gb = [&](int c) __attribute__((always_inline)) {  // prep wave 1
    const int64_t r = chunk_t0(c) + min(lane, chunk_len(c) - 1);
    gr = p.g[r * p.h_v + h];
    br = p.beta[r * p.h_v + h];
  };

  // the blocks of Tb and P~ above the diagonal blocks: zero for good
  auto zero_upper = [&](unsigned char* pb) __attribute__((always_inline)) {
    constexpr int NUP = NT * (NT - 1) / 2 * 32;  // 16-byte pieces of one matrix
    for (int e = lt; e < 2 * NUP; e += NLD) {
      const int m = e / NUP;
      int k = (e % NUP) / 32, mt = 0;
      while (k >= NT - 1 - mt) { k -= NT - 1 - mt; ++mt; }
      const int tj = mt + 1 + k, rr = (e % 32) / 2, hf = e % 2;
      *reinterpret_cast<uint4*>(pb + (m ? L::pP : L::pTb) + SC::off(mt * 16 + rr, (tj * 16 + 8 * hf) * 2)) =
          make_uint4(0u, 0u, 0u, 0u);
    }
  };

  // ------------------------------------------------ preparation, phase 1
  // prep wave 0: the NT diagonal tiles of K K^T.  A diagonal tile is
  // symmetric, so lane (g, c) holds rows 4g + i of column c; its diagonal
  // gives the row norms (lane (g, c) holds k_r . k_r, r = 16 t + c, when
  // g = c / 4, in element c % 4).  Permlane swaps (a 4x4 transpose of lane
  // row and tile) then hand lane (b, c) all of column c of tile b, from
  // which it forms column c of the block's -A and solves for column c of
  // (I + A_bb)^-1, written to sA (fp32, for the blocks below) and as Tb.
  auto diag_solve = [&](unsigned char* b, unsigned char* pb) __attribute__((always_inline)) {
    const unsigned char* K_s = b + L::rK;
    float* sc = reinterpret_cast<float*>(b + L::rSc);
    // after the transpose below, lane (bb, k) holds column k of block cb
    const int bb = g4, k = l16, cb = bb & (NT - 1);
    const int j = 16 * cb + k;
    f32x4 col[4];
#pragma unroll
    for (int t = 0; t < NT; ++t) col[t] = gram(K_s, K_s, t, t);
#pragma unroll
    for (int t = NT; t < 4; ++t) col[t] = col[t - NT];  // two blocks: lane rows 2, 3 repeat blocks 0, 1
    {  // the row norms, for the scalings of the later steps
      const int i = l16 & 3;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const float x = i == 0 ? col[t][0] : i == 1 ? col[t][1] : i == 2 ? col[t][2] : col[t][3];
        if (g4 == (l16 >> 2)) sc[2 * C + t * 16 + l16] = p.l2norm ? rsqrtf(x + 1e-6f) : 1.0f;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float a0 = col[0][i], a1 = col[1][i], a2 = col[2][i], a3 = col[3][i];
      swap_hi32(a0, a2);
      swap_hi32(a1, a3);
      swap_odd16(a0, a1);
      swap_odd16(a2, a3);
      col[0][i] = a0; col[1][i] = a1; col[2][i] = a2; col[3][i] = a3;
    }
    // col[q][e] = k_{16 cb + 4q + e} . k_{16 cb + k}: column k of block cb.
    // Its diagonal entry gives rk_j, and the rows' rk_i come from lanes
    // (bb, i) of the same row of 16 by broadcasts (no LDS round trip for
    // the norms this wave has just formed).
    const float G2j = sc[C + j];
    float dj = col[0][0];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (4 * q + e == k) dj = col[q][e];
    const float rkj = p.l2norm ? rsqrtf(dj + 1e-6f) : 1.0f;
    float nn[16];
    auto rows = [&](auto qc) __attribute__((always_inline)) {
      constexpr int q = decltype(qc)::value;
      const float4 be = *reinterpret_cast<const float4*>(sc + 16 * cb + 4 * q);
      const float4 gg = *reinterpret_cast<const float4*>(sc + C + 16 * cb + 4 * q);
      float rk[4];
      row_bcast4<q>(rk, rkj);
      const float bq[4] = {be.x, be.y, be.z, be.w}, gq[4] = {gg.x, gg.y, gg.z, gg.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * q + e;  // row 16 cb + i; e^{G_i - G_j} <= 1 where kept (i > k)
        const float a = bq[e] * rk[e] * rkj * __builtin_amdgcn_exp2f(gq[e] - G2j) * col[q][e];
        nn[i] = (p.erase && i > k) ? -a : 0.f;
      }
    };
    rows(std::integral_constant<int, 0>{});
    rows(std::integral_constant<int, 1>{});
    rows(std::integral_constant<int, 2>{});
    rows(std::integral_constant<int, 3>{});
    float t[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) t[i] = i == k ? 1.f : 0.f;
    subst16(t, nn);
    if (bb < NT) {  // Tb's diagonal blocks follow in phase 2
      float* out = sA + 16 * bb * LDF + j;
#pragma unroll
      for (int i = 0; i < 16; ++i) out[i * LDF] = t[i];
    }
  };
  // prep waves 1-3: their tiles below the diagonal blocks, K K^T and Q K^T
  // at the same (mt, tj) sharing one decay
  auto pairs = [&](const unsigned char* b, unsigned char* pb, auto pw) __attribute__((always_inline)) {
    constexpr int PW = decltype(pw)::value;
    const unsigned char* K_s = b + L::rK;
    const unsigned char* Q_s = b + L::rQ;
    const float* sc = reinterpret_cast<const float*>(b + L::rSc);
    unsigned char* P_s = pb + L::pP;
#pragma unroll
    for (int o = 0; o < pairs_of<NT>(PW); ++o) {
      const TilePair tp = pair_at<NT>(PW, o);
      const int mt = tp.mt, tj = tp.tj;
      const f32x4 kk = gram(K_s, K_s, mt, tj);
      const f32x4 qk = gram(K_s, Q_s, mt, tj);
      float w[4];
      decay(sc, mt, tj, true, w);
      const int r = mt * 16 + l16, j0 = tj * 16 + 4 * g4;
      *reinterpret_cast<float4*>(sA + r * LDF + j0) = make_float4(w[0] * kk[0], w[1] * kk[1], w[2] * kk[2], w[3] * kk[3]);
      put_p(P_s, mt, tj, w, qk);
    }
  };
  auto prep_phase1 = [&](unsigned char* b, unsigned char* pb) __attribute__((always_inline)) {
    if (pi == 0) {
      __builtin_amdgcn_s_setprio(3);
      diag_solve(b, pb);
      __builtin_amdgcn_s_setprio(0);
    }
    else if (pi == 1) pairs(b, pb, std::integral_constant<int, 1>{});
    else if (pi == 2) {
      pairs(b, pb, std::integral_constant<int, 2>{});
      if constexpr (W) {
        // scale rq of each row for the outputs (once, rather than in every
        // chain wave): lane r sums |q_r|^2 over its raw row
        if (lane < C) {
          const unsigned char* Q_s = b + L::rQ;
          float qq = 0.f;
#pragma unroll
          for (int j = 0; j < D / 8; ++j) {
            const uint4 w = *reinterpret_cast<const uint4*>(Q_s + SK::off(lane, j * 16));
            const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
              qq = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, ww[e]), __builtin_bit_cast(bf16x2, ww[e]), qq, false);
          }
          reinterpret_cast<float*>(pb + L::pVec)[5 * C + lane] = p.scale * (p.l2norm ? rsqrtf(qq + 1e-6f) : 1.0f);
        }
      }
    }
    else pairs(b, pb, std::integral_constant<int, 3>{});
  };
  // output waves (chain waves of a wide workgroup): the diagonal tiles of
  // Q K^T (tiles ow, ow + NC, ...)
  auto prep1_pdiag = [&](const unsigned char* b, unsigned char* pb, int ow) __attribute__((always_inline)) {
    const unsigned char* K_s = b + L::rK;
    const unsigned char* Q_s = b + L::rQ;
    const float* sc = reinterpret_cast<const float*>(b + L::rSc);
    if constexpr (W) {
      // chain waves: a loop over the wave's tiles with the tile index known
      // only at run time, so that their offsets are formed here instead of
      // being held in registers across the chunk loop
      int t0 = ow, ln = lane;
      asm volatile("" : "+s"(t0), "+v"(ln));
      const int lx = ln & 15, gx = ln >> 4;
      for (int t = t0; t < NT; t += NC) {
        f32x4 qk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < DKS; ++s)
          M::mma(qk, frag_row_s<T, SK>(K_s, t * 16 + lx, 32 * s + 8 * gx, false),
                 frag_row_s<T, SK>(Q_s, t * 16 + lx, 32 * s + 8 * gx, false), false);
        float w[4];
        decay_l(sc, t, t, false, w, lx, gx);
        put_p_l(pb + L::pP, t, t, w, qk, lx, gx);
      }
    } else {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t % NC != ow) continue;
        const f32x4 qk = gram(K_s, Q_s, t, t);
        float w[4];
        decay(sc, t, t, false, w);
        put_p(pb + L::pP, t, t, w, qk);
      }
    }
  };

  // ------------------------------------------------ preparation, phase 2
  // The blocks of T below the diagonal blocks follow from (I + A) T = I:
  //   T_10 = -T_11 A_10 T_00,  T_32 = -T_33 A_32 T_22,
  //   X_ij = A_i0 T_0j + A_i1 T_1j,
  //   T_2j = -T_22 X_2j,  T_3j = -T_33 (X_3j + A_32 T_2j)      (j = 0, 1)
  // on bf16 MFMA (16x16x32, k over two 16-blocks; a block above the
  // diagonal enters as zero; A's blocks take their row scaling beta_r rk_r
  // and column scaling rk_j as they are converted), each written as a block
  // of Tb = T diag(beta).  Prep wave 1 forms T_32 (T_10 when there are two
  // blocks), wave 2 column block 0 (T_10, T_20, T_30), wave 3 column block 1
  // (T_21, T_31), wave 0 the row scalars.
  auto prep_phase2 = [&](const unsigned char* b, unsigned char* pb) __attribute__((always_inline)) {
    const float* sc = reinterpret_cast<const float*>(b + L::rSc);
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    auto colb = [&](int bi, int bj) __attribute__((always_inline)) {  // accumulator layout: rows 4g + i, column c
      const float* a = sA + (16 * bi + 4 * g4) * LDF + 16 * bj + l16;
      return f32x4{a[0], a[LDF], a[2 * LDF], a[3 * LDF]};
    };
    // A fragment, rows 16 bi + l16 over blocks bj0 | bj1 (bj1 < 0: zeros),
    // of T (scaled = false) or of A (from A~, scaled)
    auto rowf = [&](int bi, int bj0, int bj1, bool scaled) __attribute__((always_inline)) {
      const int r = 16 * bi + l16;
      const float* a = sA + r * LDF + 4 * g4;
      float4 x = *reinterpret_cast<const float4*>(a + 16 * bj0);
      float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
      if (bj1 >= 0) y = *reinterpret_cast<const float4*>(a + 16 * bj1);
      if (scaled) {
        const float fa = p.erase ? sc[r] * sc[2 * C + r] : 0.f;
        const float4 k0 = *reinterpret_cast<const float4*>(sc + 2 * C + 16 * bj0 + 4 * g4);
        x = make_float4(fa * k0.x * x.x, fa * k0.y * x.y, fa * k0.z * x.z, fa * k0.w * x.w);
        if (bj1 >= 0) {
          const float4 k1 = *reinterpret_cast<const float4*>(sc + 2 * C + 16 * bj1 + 4 * g4);
          y = make_float4(fa * k1.x * y.x, fa * k1.y * y.y, fa * k1.z * y.z, fa * k1.w * y.w);
        }
      }
      return __builtin_bit_cast(frag, make_uint4(pack_bf16x2(x.x, x.y), pack_bf16x2(x.z, x.w),
                                                 pack_bf16x2(y.x, y.y), pack_bf16x2(y.z, y.w)));
    };
    // block (bi, bj) of Tb from T in accumulator layout
    auto put_tb = [&](int bi, int bj, const f32x4& t) __attribute__((always_inline)) {
      unsigned char* tb = pb + L::pTb;
      const float bc = sc[16 * bj + l16];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<__bf16*>(tb + SC::off(16 * bi + 4 * g4 + i, (16 * bj + l16) * 2)) = (__bf16)(t[i] * bc);
    };
    // Every operand is read before the first product (one LDS round trip);
    // the blocks are written after the last.
    // T_{i+1, i} = -T_{i+1, i+1} A_{i+1, i} T_ii
    auto level1 = [&](const frag& a, const f32x4& tii, const frag& tnext) __attribute__((always_inline)) {
      f32x4 x = zero, l = zero;
      M::mma(x, a, M::acc(tii, zero), false);
      M::mma(l, tnext, M::acc(x, zero), false);
      return -l;
    };
    // T_2j = -T_22 X_2j,  T_3j = -T_33 (X_3j + A_32 T_2j)
    auto lower_pair = [&](const frag& t22, const frag& a32, const frag& t33, const f32x4& x2, f32x4 x3,
                          f32x4& t2, f32x4& t3) __attribute__((always_inline)) {
      t2 = zero;
      t3 = zero;
      M::mma(t2, t22, M::acc(x2, zero), false);
      t2 = -t2;
      M::mma(x3, a32, M::acc(t2, zero), false);
      M::mma(t3, t33, M::acc(x3, zero), false);
      t3 = -t3;
    };
    if constexpr (NT == 2) {
      if (pi == 1) {
        const frag a10 = rowf(1, 0, -1, true), t11 = rowf(1, 1, -1, false);
        const f32x4 t00 = colb(0, 0);
        put_tb(1, 0, level1(a10, t00, t11));
      }
    } else {
      if (pi == 1) {
        const frag a32 = rowf(3, 2, -1, true), t33 = rowf(3, 3, -1, false);
        const f32x4 t22 = colb(2, 2);
        put_tb(3, 2, level1(a32, t22, t33));
      } else if (pi == 2) {
        const frag a10 = rowf(1, 0, -1, true), t11 = rowf(1, 1, -1, false);
        const frag a2 = rowf(2, 0, 1, true), a3 = rowf(3, 0, 1, true);
        const frag t22 = rowf(2, 2, -1, false), a32 = rowf(3, 2, -1, true), t33 = rowf(3, 3, -1, false);
        const f32x4 t00 = colb(0, 0);
        const f32x4 t10 = level1(a10, t00, t11);
        const frag bt = M::acc(t00, t10);
        f32x4 x2 = zero, x3 = zero, t2, t3;
        M::mma(x2, a2, bt, false);
        M::mma(x3, a3, bt, false);
        lower_pair(t22, a32, t33, x2, x3, t2, t3);
        put_tb(1, 0, t10);
        put_tb(2, 0, t2);
        put_tb(3, 0, t3);
      } else if (pi == 3) {
        const frag a2 = rowf(2, 1, -1, true), a3 = rowf(3, 1, -1, true);
        const frag t22 = rowf(2, 2, -1, false), a32 = rowf(3, 2, -1, true), t33 = rowf(3, 3, -1, false);
        const frag bt = M::acc(colb(1, 1), zero);
        f32x4 x2 = zero, x3 = zero, t2, t3;
        M::mma(x2, a2, bt, false);
        M::mma(x3, a3, bt, false);
        lower_pair(t22, a32, t33, x2, x3, t2, t3);
        put_tb(2, 1, t2);
        put_tb(3, 1, t3);
      }
    }
    // prep wave 0: Tb's diagonal blocks, T_bb diag(beta) from the fp32
    // blocks the diagonal solve left in sA (lane 16 bi + r: row r of block
    // bi, two 16-byte stores)
    if (pi == 0 && lane < C) {
      const int bi = lane >> 4, r = lane;
      const float* a = sA + r * LDF + 16 * bi;
      const float* bc = sc + 16 * bi;
      uint32_t w[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 t4 = *reinterpret_cast<const float4*>(a + 4 * q);
        const float4 b4 = *reinterpret_cast<const float4*>(bc + 4 * q);
        w[2 * q] = pack_bf16x2(t4.x * b4.x, t4.y * b4.y);
        w[2 * q + 1] = pack_bf16x2(t4.z * b4.z, t4.w * b4.w);
      }
      unsigned char* tb = pb + L::pTb;
      *reinterpret_cast<uint4*>(tb + SC::off(r, 32 * bi)) = make_uint4(w[0], w[1], w[2], w[3]);
      *reinterpret_cast<uint4*>(tb + SC::off(r, 32 * bi + 16)) = make_uint4(w[4], w[5], w[6], w[7]);
    }
    // row scalars: gamma rk (0 without the erase: R = V), gamma, e rk,
    // gamma_last (G of padding rows equals the last row's), rk
    if (pi == 0 && lane < C) {
      float* vec = reinterpret_cast<float*>(pb + L::pVec);
      const float G = sc[C + lane], Gl = sc[2 * C - 1], eg = __builtin_amdgcn_exp2f(G), rk = sc[2 * C + lane];
      vec[lane] = p.erase ? eg * rk : 0.f;
      vec[C + lane] = eg;
      vec[2 * C + lane] = __builtin_amdgcn_exp2f(Gl - G) * rk;
      vec[3 * C + lane] = __builtin_amdgcn_exp2f(Gl);
      vec[4 * C + lane] = rk;
    }
  };

  // ------------------------------------------------------------ prologue
  if (nch > 0 && W) {
    if (prepw) {
      zero_upper(prp0);
      zero_upper(prp1);
      dma_raw(0, raw0);
      if (pi == 1) {
        load_gb(0);
        store_sc(0, raw0);
      }
    }
    barrier_vm<0>();  // raw chunk 0 has landed
    if (prepw) prep_phase1(raw0, prp0);
    if (chain) prep1_pdiag(raw0, prp0, wave);
    barrier_vm<63>();  // chunk 0's T_bb, A~ and norms complete
    if (prepw) {
      if (nch > 1) {
        dma_raw(1, raw1);
        if (pi == 1) load_gb(1);
      }
      prep_phase2(raw0, prp0);
      if (nch > 1 && pi == 1) store_sc(1, raw1);
      if (nch > 2 && pi == 1) load_gb(2);
    }
  } else if (nch > 0) {
    if (prepw) {
      zero_upper(prp0);
      zero_upper(prp1);
      load_raw(0);
      store_raw(0, raw0);
      if (nch > 1) load_raw(1);
    }
    barrier_vm<63>();  // raw chunk 0 visible
    if (prepw) prep_phase1(raw0, prp0);
    if (outw) prep1_pdiag(raw0, prp0, wave - NC);
    barrier_vm<63>();  // chunk 0's T_bb, A~ and norms complete
    if (prepw) {
      prep_phase2(raw0, prp0);
      if (nch > 1) {
        store_raw(1, raw1);
        if (nch > 2) load_raw(2);
      }
    }
  }
  if constexpr (W) {
    if (chain) {
      // ------------------------------------------------ wide: chain waves
      // Columns 32 wave .. 32 wave + 31 of the state, S^T in CT x DT
      // accumulator tiles as in the narrow chain.  Per chunk c, before B1:
      // X1 = K S^T with Y^T = S Q^T, R, U = Tb R and the state update; after
      // B1, O^T = scale rq (gamma Y^T + (U diag(rk))^T P~^T), stored, chunk
      // c+1's diagonal Q K^T tiles and any emitted state.
      f32x4 st[CT][DT];
      const int sslot = p.state_idx ? as_const(p.state_idx)[n] : n;
      // element offset of the lane's tile (ct, dt) inside a head's d x d
      // state (row = d_v column), from the lane's base offset lb.  The base
      // passes through an empty asm where it is used, so the compiler forms
      // the addresses there instead of holding all of them across the loop.
      const int lb0 = (16 * CT * wave + l16) * D + 8 * g4;
      auto toff = [&](int lb, int ct, int dt) __attribute__((always_inline)) {
        return (uint32_t)(lb + 16 * ct * D + pidx<DT>(dt, 0));
      };
      auto opaque = [](int x) __attribute__((always_inline)) {
        asm volatile("" : "+v"(x));
        return x;
      };
      // uniform bases with 32-bit lane offsets (SGPR base + VGPR offset
      // addressing: no 64-bit address per tile)
      const size_t sbase = ((size_t)sslot * p.h_v + h) * D * D;
      auto sptr = [&](void* base, size_t e) __attribute__((always_inline)) {
        return p.state_bf16 ? (void*)(reinterpret_cast<__bf16*>(base) + e) : (void*)(reinterpret_cast<float*>(base) + e);
      };
      const int erow = p.emit_every > 0 ? plan.erow(n) : 0;
      const int o_stride = p.h_v * D;
      T* og = reinterpret_cast<T*>(p.o) + (int64_t)h * D;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          st[ct][dt] = p.initial_state ? load_state4(sptr(const_cast<void*>(p.initial_state), sbase), toff(lb0, ct, dt), p.state_bf16)
                                       : f32x4{0.f, 0.f, 0.f, 0.f};
      barrier_vm<63>();  // chunk 0's preparation and chunk 1's rows are visible
      // the chunk's LDS buffers pass through an empty asm: every address in
      // them is then formed in the step rather than held across the loop
      auto launder = [](const unsigned char* x) __attribute__((always_inline)) {
        auto q = (__attribute__((address_space(3))) const unsigned char*)x;
        asm volatile("" : "+v"(q));
        return (const unsigned char*)q;
      };
      auto step = [&](int c, const unsigned char* rb0, const unsigned char* pb0, const unsigned char* rn,
                      unsigned char* pn) __attribute__((always_inline)) {
        const unsigned char* rb = launder(rb0);
        const unsigned char* pb = launder(pb0);
        const unsigned char* K_t = rb + L::rK;
        const unsigned char* Q_t = rb + L::rQ;
        const unsigned char* V_t = rb + L::rV;
        const unsigned char* Tb_t = pb + L::pTb;
        const unsigned char* P_t = pb + L::pP;
        const float* vec = reinterpret_cast<const float*>(pb + L::pVec);
        // X1 = K S^T and Y^T = S Q^T (raw q): one bf16 fragment of S is the
        // B operand of the first and the A operand of the second
        f32x4 x1[CT][NT], o[CT][NT];
#pragma unroll
        for (int mt = 0; mt < NT; ++mt)
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) x1[ct][mt] = o[ct][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < DKS; ++s) {
          frag ak[NT], bq[NT];
#pragma unroll
          for (int mt = 0; mt < NT; ++mt) {
            ak[mt] = frag_row_s<T, SK>(K_t, pidx<NT>(mt, l16), 32 * s + 8 * g4, false);
            bq[mt] = frag_row_s<T, SK>(Q_t, pidx<NT>(mt, l16), 32 * s + 8 * g4, false);
          }
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) {
            const frag bs = M::acc(st[ct][2 * s], st[ct][2 * s + 1]);
#pragma unroll
            for (int mt = 0; mt < NT; ++mt) {
              M::mma(x1[ct][mt], ak[mt], bs, false);
              M::mma(o[ct][mt], bs, bq[mt], false);
            }
          }
        }
        // R = V - diag(gamma rk) X1, V[token pidx(mt, 4g) + e][column] by
        // one transposing read per tile
#pragma unroll
        for (int mt = 0; mt < NT; ++mt) {
          const float4 vq = *reinterpret_cast<const float4*>(vec + pidx<NT>(mt, 4 * g4));
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) {
            const int r0 = pidx<NT>(mt, 4 * g4);
            const uint2 vw = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(
                __attribute__((address_space(3))) unsigned char*)(V_t + SV::off(r0 + (l16 >> 2),
                                                                                (16 * (CT * wave + ct) + 4 * (l16 & 3)) * 2))));
            x1[ct][mt][0] = bf16_lo(vw.x) - vq.x * x1[ct][mt][0];
            x1[ct][mt][1] = bf16_hi(vw.x) - vq.y * x1[ct][mt][1];
            x1[ct][mt][2] = bf16_lo(vw.y) - vq.z * x1[ct][mt][2];
            x1[ct][mt][3] = bf16_hi(vw.y) - vq.w * x1[ct][mt][3];
          }
        }
        // U = Tb R
        f32x4 u[CT][NT];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
          for (int mt = 0; mt < NT; ++mt) u[ct][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          frag at[NT];
#pragma unroll
          for (int mt = 0; mt < NT; ++mt) at[mt] = frag_row_s<T, SC>(Tb_t, pidx<NT>(mt, l16), 32 * s + 8 * g4, false);
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) {
            const frag bs = M::acc(x1[ct][2 * s], x1[ct][2 * s + 1]);
#pragma unroll
            for (int mt = 0; mt < NT; ++mt) M::mma(u[ct][mt], at[mt], bs, false);
          }
        }
        // (U diag(rk))^T as A fragments of the output product and
        // U' = diag(e rk) U as B fragments of the state update
        frag au[KS][CT], bu[KS][CT];
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const float4 r0 = *reinterpret_cast<const float4*>(vec + 4 * C + pidx<NT>(2 * s, 4 * g4));
          const float4 r1 = *reinterpret_cast<const float4*>(vec + 4 * C + pidx<NT>(2 * s + 1, 4 * g4));
          const float4 e0 = *reinterpret_cast<const float4*>(vec + 2 * C + pidx<NT>(2 * s, 4 * g4));
          const float4 e1 = *reinterpret_cast<const float4*>(vec + 2 * C + pidx<NT>(2 * s + 1, 4 * g4));
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) {
            const f32x4 a = u[ct][2 * s], b = u[ct][2 * s + 1];
            au[s][ct] = M::acc(f32x4{a[0] * r0.x, a[1] * r0.y, a[2] * r0.z, a[3] * r0.w},
                               f32x4{b[0] * r1.x, b[1] * r1.y, b[2] * r1.z, b[3] * r1.w});
            bu[s][ct] = M::acc(f32x4{a[0] * e0.x, a[1] * e0.y, a[2] * e0.z, a[3] * e0.w},
                               f32x4{b[0] * e1.x, b[1] * e1.y, b[2] * e1.z, b[3] * e1.w});
          }
        }
        // S^T <- gamma_last S^T + K^T U' (the raw buffer is refilled after B1)
        const float gl = vec[3 * C];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) st[ct][dt] *= gl;
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const frag kt = frag_kt<T, L::RBK, DT>(K_t, dt, 32 * s + 8 * g4, l16, false);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) M::mma(st[ct][dt], kt, bu[s][ct], false);
          }
        barrier_vm<63>();  // B1
        // O^T = scale rq (gamma Y^T + (U diag(rk))^T P~^T)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const float gm = vec[C + pidx<NT>(nt, l16)];
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) o[ct][nt] *= gm;
        }
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          frag bp[NT];
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) bp[nt] = frag_row_s<T, SC>(P_t, pidx<NT>(nt, l16), 32 * s + 8 * g4, false);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) M::mma(o[ct][nt], au[s][ct], bp[nt], false);
        }
        const int Lc = chunk_len(c);
        T* oc = og + chunk_t0(c) * (int64_t)o_stride;
        const int l16s = opaque(l16);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int tok = pidx<NT>(nt, l16s);
          const float f = vec[5 * C + tok];
          if (tok < Lc) {
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
              *reinterpret_cast<uint2*>(oc + (uint32_t)(tok * o_stride + 16 * (CT * wave + ct) + 4 * g4)) =
                  make_uint2(pack_bf16x2(f * o[ct][nt][0], f * o[ct][nt][1]), pack_bf16x2(f * o[ct][nt][2], f * o[ct][nt][3]));
          }
        }
        // chunk c+1's diagonal Q K^T tiles
        if (c + 1 < nch) prep1_pdiag(rn, pn, wave);
        // the state after every emit_every-th whole chunk inside the sequence
        // (last, when the output tiles are no longer held)
        if (p.emit_every > 0 && (c + 1) % p.emit_every == 0 && chunk_t0(c) + C < seq_end) {
          const size_t dst = ((size_t)(erow + (c + 1) / p.emit_every - 1) * p.h_v + h) * D * D;
          const int lb = opaque(lb0);
#pragma unroll
          for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
              store_state4(sptr(p.chunk_states, dst), toff(lb, ct, dt), st[ct][dt], p.state_bf16);
        }
        barrier_vm<63>();  // B2
      };
      for (int c = 0; c < nch; c += 2) {
        step(c, raw0, prp0, raw1, prp1);
        if (c + 1 < nch) step(c + 1, raw1, prp1, raw0, prp0);
      }
      if (p.final_state) {
        const int lb = opaque(lb0);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
            store_state4(sptr(p.final_state, sbase), toff(lb, ct, dt), st[ct][dt], p.state_bf16);
      }
    } else {
      // ------------------------------------------------- wide: prep waves
      // rb: chunk c (free after B1, then filled with chunk c+2 by direct
      // loads that land before B2); rn, pn: chunk c+1.  Prep wave 1 loads g
      // and beta a step ahead of their use (chunk c+3 in step c), so their
      // latency is spent across a barrier.
      barrier_vm<0>();  // chunk 1's rows have landed
      auto step = [&](int c, unsigned char* rb, unsigned char* rn, unsigned char* pn) __attribute__((always_inline)) {
        if (pi != 0) touch(c + 2);
        if (c + 1 < nch) prep_phase1(rn, pn);
        barrier_vm<63>();  // B1
        if (c + 2 < nch) dma_raw(c + 2, rb);
        if (c + 1 < nch) prep_phase2(rn, pn);
        if (pi == 1) {
          if (c + 2 < nch) store_sc(c + 2, rb);
          if (c + 3 < nch) load_gb(c + 3);
          barrier_vm<2>();  // B2: chunk c+2 has landed; g and beta stay in flight
        } else {
          barrier_vm<0>();  // B2: chunk c+2 has landed
        }
      };
      for (int c = 0; c < nch; c += 2) {
        step(c, raw0, raw1, prp1);
        if (c + 1 < nch) step(c + 1, raw1, raw0, prp0);
      }
      asm volatile("" ::"v"(tv0), "v"(tv1), "v"(tv2), "v"(tv3));
    }
  } else {
  if (chain) {
    // ---------------------------------------------------------- chain waves
    // S^T (d_k x this wave's 16 CT columns) in CT x DT accumulator tiles;
    // row 4g+i of tile dt is d_k index pidx<DT>(dt, 4g+i)
    auto colof = [&](int ct) __attribute__((always_inline)) { return 16 * (CT * wave + ct) + l16; };
    f32x4 st[CT][DT];
    const int sslot = p.state_idx ? as_const(p.state_idx)[n] : n;
    auto srow = [&](int ct) __attribute__((always_inline)) {
      return (((size_t)sslot * p.h_v + h) * D + (size_t)(blk * L::cols + colof(ct))) * D;
    };
    auto wrow = [&](int ct) __attribute__((always_inline)) {
      return ((size_t)h * D + (size_t)(blk * L::cols + colof(ct))) * D;
    };
    const int erow = p.emit_every > 0 ? plan.erow(n) : 0;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        st[ct][dt] = p.initial_state ? load_state4(p.initial_state, srow(ct) + pidx<DT>(dt, 4 * g4), p.state_bf16)
                                     : f32x4{0.f, 0.f, 0.f, 0.f};
    auto publish_state = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int u = 0; u < DT / 2; ++u)
          *reinterpret_cast<frag*>(sS + SS::off(colof(ct), (32 * u + 8 * g4) * 2)) = M::acc(st[ct][2 * u], st[ct][2 * u + 1]);
    };
    publish_state();
    barrier_vm<63>();  // the initial state and chunk 0's preparation are visible
    auto step = [&](int c, const unsigned char* rb, const unsigned char* pb) __attribute__((always_inline)) {
      const unsigned char* K_t = rb + L::rK;
      const unsigned char* V_t = rb + L::rV;
      const unsigned char* Tb_t = pb + L::pTb;
      const float* vec = reinterpret_cast<const float*>(pb + L::pVec);
      // V[token pidx(mt, 4g) + e][column] by one transposing read per tile
      uint2 vw[CT][NT];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int mt = 0; mt < NT; ++mt) {
          const int r0 = pidx<NT>(mt, 4 * g4);
          vw[ct][mt] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(
              __attribute__((address_space(3))) unsigned char*)(V_t + SV::off(r0 + (l16 >> 2),
                                                                              (16 * (CT * wave + ct) + 4 * (l16 & 3)) * 2))));
        }
      frag at[KS][NT];
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int mt = 0; mt < NT; ++mt) at[s][mt] = frag_row_s<T, SC>(Tb_t, pidx<NT>(mt, l16), 32 * s + 8 * g4, false);
      // X1 = K S^T
      f32x4 x1[CT][NT];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int mt = 0; mt < NT; ++mt) x1[ct][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < DKS; ++s) {
        frag ak[NT];
#pragma unroll
        for (int mt = 0; mt < NT; ++mt) ak[mt] = frag_row_s<T, SK>(K_t, pidx<NT>(mt, l16), 32 * s + 8 * g4, false);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const frag bs = M::acc(st[ct][2 * s], st[ct][2 * s + 1]);
#pragma unroll
          for (int mt = 0; mt < NT; ++mt) M::mma(x1[ct][mt], ak[mt], bs, false);
        }
      }
      // R = V - diag(gamma rk) X1
#pragma unroll
      for (int mt = 0; mt < NT; ++mt) {
        const float4 vq = *reinterpret_cast<const float4*>(vec + pidx<NT>(mt, 4 * g4));
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          x1[ct][mt][0] = bf16_lo(vw[ct][mt].x) - vq.x * x1[ct][mt][0];
          x1[ct][mt][1] = bf16_hi(vw[ct][mt].x) - vq.y * x1[ct][mt][1];
          x1[ct][mt][2] = bf16_lo(vw[ct][mt].y) - vq.z * x1[ct][mt][2];
          x1[ct][mt][3] = bf16_hi(vw[ct][mt].y) - vq.w * x1[ct][mt][3];
        }
      }
      // U = Tb R
      f32x4 u[CT][NT];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int mt = 0; mt < NT; ++mt) u[ct][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const frag bs = M::acc(x1[ct][2 * s], x1[ct][2 * s + 1]);
#pragma unroll
          for (int mt = 0; mt < NT; ++mt) M::mma(u[ct][mt], at[s][mt], bs, false);
        }
      // publish U as bf16 rows [column][token]
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int s = 0; s < KS; ++s)
          *reinterpret_cast<frag*>(sU + SU::off(colof(ct), (32 * s + 8 * g4) * 2)) = M::acc(u[ct][2 * s], u[ct][2 * s + 1]);
      // U' = diag(e rk) U
#pragma unroll
      for (int mt = 0; mt < NT; ++mt) {
        const float4 vq = *reinterpret_cast<const float4*>(vec + 2 * C + pidx<NT>(mt, 4 * g4));
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          u[ct][mt][0] *= vq.x; u[ct][mt][1] *= vq.y; u[ct][mt][2] *= vq.z; u[ct][mt][3] *= vq.w;
        }
      }
      // S^T <- gamma_last S^T + K^T U', before B1 (the raw buffer is refilled
      // after it); the new state is published after B1, once the output
      // waves are done with the old one
      const float gl = vec[3 * C];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) st[ct][dt] *= gl;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        frag bs[CT];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) bs[ct] = M::acc(u[ct][2 * s], u[ct][2 * s + 1]);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const frag kt = frag_kt<T, L::RBK, DT>(K_t, dt, 32 * s + 8 * g4, l16, false);
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) M::mma(st[ct][dt], kt, bs[ct], false);
        }
      }
      barrier_vm<63>();  // B1
      // the state after every emit_every-th whole chunk inside the sequence
      if (p.emit_every > 0 && (c + 1) % p.emit_every == 0 && chunk_t0(c) + C < seq_end) {
        const size_t dst = (size_t)(erow + (c + 1) / p.emit_every - 1) * p.h_v * D * D;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
            store_state4(p.chunk_states, dst + wrow(ct) + pidx<DT>(dt, 4 * g4), st[ct][dt], p.state_bf16);
      }
      publish_state();
      barrier_vm<63>();  // B2
    };
    for (int c = 0; c < nch; c += 2) {
      step(c, raw0, prp0);
      if (c + 1 < nch) step(c + 1, raw1, prp1);
    }
    if (p.final_state) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          store_state4(p.final_state, srow(ct) + pidx<DT>(dt, 4 * g4), st[ct][dt], p.state_bf16);
    }
  } else if (outw) {
    // --------------------------------------------------------- output waves
    const int ow = wave - NC;
    const int64_t o_stride = (int64_t)p.h_v * D;
    T* og = reinterpret_cast<T*>(p.o) + (int64_t)h * D + blk * L::cols + 4 * g4;
    auto colr = [&](int ct) __attribute__((always_inline)) { return 16 * (CT * ow + ct) + l16; };
    barrier_vm<63>();  // the initial state and chunk 0's preparation are visible
    // rb, pb: chunk c; rn, pn: chunk c+1 (its diagonal Q K^T tiles)
    auto step = [&](int c, const unsigned char* rb, const unsigned char* pb, const unsigned char* rn,
                    unsigned char* pn) __attribute__((always_inline)) {
      const unsigned char* Q_t = rb + L::rQ;
      const unsigned char* P_t = pb + L::pP;
      const float* vec = reinterpret_cast<const float*>(pb + L::pVec);
      // O^T tile (ct, nt): rows 4g + i = columns 16 (CT ow + ct) + 4g + i,
      // column l16 = token pidx(nt, l16).  First Y^T = S Q^T (raw q), scaled
      // by gamma; the lane's part of |q|^2 comes from the same fragments
      f32x4 o[CT][NT];
      float qq[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        qq[nt] = 0.f;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) o[ct][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int s = 0; s < DKS; ++s) {
        frag as[CT];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) as[ct] = frag_row_s<T, SS>(sS, colr(ct), 32 * s + 8 * g4, false);
        frag bq[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) bq[nt] = frag_row_s<T, SK>(Q_t, pidx<NT>(nt, l16), 32 * s + 8 * g4, false);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) M::mma(o[ct][nt], as[ct], bq[nt], false);
          const uint4 w = __builtin_bit_cast(uint4, bq[nt]);
          const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int j = 0; j < 4; ++j)
            qq[nt] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, ww[j]), __builtin_bit_cast(bf16x2, ww[j]), qq[nt], false);
        }
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const float gm = vec[C + pidx<NT>(nt, l16)];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) o[ct][nt] *= gm;
        // sum over the four lane rows (lanes l, l ^ 16, l ^ 32, l ^ 48)
        float a = qq[nt], b = qq[nt];
        swap_hi32(a, b);
        a += b;
        b = a;
        swap_odd16(a, b);
        qq[nt] = a + b;
      }
      if (c + 1 < nch) prep1_pdiag(rn, pn, ow);
      barrier_vm<63>();  // B1: U is published
      // O^T += (U diag(rk))^T P~^T
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const float4 r0 = *reinterpret_cast<const float4*>(vec + 4 * C + 32 * s + 8 * g4);
        const float4 r1 = *reinterpret_cast<const float4*>(vec + 4 * C + 32 * s + 8 * g4 + 4);
        frag au[CT];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const uint4 uw = __builtin_bit_cast(uint4, frag_row_s<T, SU>(sU, colr(ct), 32 * s + 8 * g4, false));
          au[ct] = __builtin_bit_cast(frag, make_uint4(
              pack_bf16x2(bf16_lo(uw.x) * r0.x, bf16_hi(uw.x) * r0.y), pack_bf16x2(bf16_lo(uw.y) * r0.z, bf16_hi(uw.y) * r0.w),
              pack_bf16x2(bf16_lo(uw.z) * r1.x, bf16_hi(uw.z) * r1.y), pack_bf16x2(bf16_lo(uw.w) * r1.z, bf16_hi(uw.w) * r1.w)));
        }
        frag bp[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) bp[nt] = frag_row_s<T, SC>(P_t, pidx<NT>(nt, l16), 32 * s + 8 * g4, false);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) M::mma(o[ct][nt], au[ct], bp[nt], false);
      }
      const int Lc = chunk_len(c);
      T* oc = og + chunk_t0(c) * o_stride;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int tok = pidx<NT>(nt, l16);
        const float f = p.scale * (p.l2norm ? rsqrtf(qq[nt] + 1e-6f) : 1.0f);
        if (tok < Lc) {
#pragma unroll
          for (int ct = 0; ct < CT; ++ct)
            *reinterpret_cast<uint2*>(oc + (int64_t)tok * o_stride + 16 * (CT * ow + ct)) =
                make_uint2(pack_bf16x2(f * o[ct][nt][0], f * o[ct][nt][1]), pack_bf16x2(f * o[ct][nt][2], f * o[ct][nt][3]));
        }
      }
      barrier_vm<63>();  // B2
    };
    for (int c = 0; c < nch; c += 2) {
      step(c, raw0, prp0, raw1, prp1);
      if (c + 1 < nch) step(c + 1, raw1, prp1, raw0, prp0);
    }
  } else {
    // ---------------------------------------------------------- prep waves
    barrier_vm<63>();  // the initial state and chunk 0's preparation are visible
    // rb: chunk c (free after B1), then chunk c+2; rn, pn: chunk c+1
    auto step = [&](int c, unsigned char* rb, unsigned char* rn, unsigned char* pn) __attribute__((always_inline)) {
      if (c + 1 < nch) prep_phase1(rn, pn);
      barrier_vm<63>();  // B1
      if (c + 1 < nch) prep_phase2(rn, pn);
      if (c + 2 < nch) {
        store_raw(c + 2, rb);
        if (c + 3 < nch) load_raw(c + 3);
      }
      barrier_vm<63>();  // B2: loads of the chunk after next stay in flight
    };
    for (int c = 0; c < nch; c += 2) {
      step(c, raw0, raw1, prp1);
      if (c + 1 < nch) step(c + 1, raw1, raw0, prp0);
    }
  }
  }
}

#define GDN_FUSED(D, C) \
  template __global__ void fused_kernel<D, C, 1, 1, false>(PrefillParams, const unsigned char*); \
  template __global__ void fused_kernel<D, C, 2, 1, false>(PrefillParams, const unsigned char*); \
  template __global__ void fused_kernel<D, C, 2, 2, false>(PrefillParams, const unsigned char*); \
  template __global__ void fused_kernel<D, C, D / 32, 2, true>(PrefillParams, const unsigned char*);
GDN_FUSED(64, 32) GDN_FUSED(64, 64) GDN_FUSED(128, 32) GDN_FUSED(128, 64)
#undef GDN_FUSED

// ------------------------------------------------------------------ host
constexpr int kLdsMax = 160 * 1024;
// scan workgroup shape: kScanWaves waves, each owning kScanTiles 16-column
// tiles of the state (64 d_v columns per workgroup)
#ifndef GDN_SCAN_WAVES
#define GDN_SCAN_WAVES 4
#endif
#ifndef GDN_SCAN_TILES
#define GDN_SCAN_TILES 1
#endif
constexpr int kScanWaves = GDN_SCAN_WAVES;
constexpr int kScanTiles = GDN_SCAN_TILES;

// bf16 runs the split-role scan, fp32 the four-wave scan
template <typename T, int D, int C>
constexpr int scan_lds_bytes() {
  if constexpr (sizeof(T) == 2) return Scan2Layout<D, C, 64>::bytes;
  else return ScanLayout<T, D, C, kScanWaves, kScanTiles>::bytes;
}

template <typename T, int D, int C>
constexpr bool fits() {
  return PrepLayout<T, D, C, 1>::bytes <= kLdsMax && scan_lds_bytes<T, D, C>() <= kLdsMax;
}

template <typename T, int D, int C, int VPW>
hipError_t launch_prep(const PrefillParams& p, unsigned char* ws, int64_t mc, hipStream_t stream) {
  using PL = PrepLayout<T, D, C, VPW>;
  if constexpr (PL::bytes > kLdsMax) {
    return hipErrorInvalidConfiguration;
  } else {
    auto prep = prep_kernel<T, D, C, VPW>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(prep),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, PL::bytes);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(prep, dim3((unsigned)mc, (unsigned)(p.h_v / VPW)), dim3(kPrepThreads * VPW), PL::bytes,
                       stream, p, ws);
    return hipGetLastError();
  }
}

// bf16 at chunk 32 and 64 runs the fused kernel (plan_kernel first with
// cu_seqlens); its workspace is the plan's arrays only
template <typename T, int C>
constexpr bool fused_path() { return sizeof(T) == 2 && C >= 32; }
// The fused kernel runs when its widest workgroups (64 columns) fill the
// chip by themselves: many (sequence, V head) pairs, where it does the least
// work per chunk.  With fewer, the serial chains of a few long sequences set
// the time, and the separate preparation and scan launches are faster.
// GDN_PREFILL_FUSED=1 or 0 forces the choice (tuning and comparison); the
// workspace query follows it.
inline bool use_fused(int io_dtype, int chunk, int n_seqs, int h_v, int d) {
  const char* e = std::getenv("GDN_PREFILL_FUSED");  // read per call: tests switch it in-process
  const int forced = e && e[0] ? (e[0] == '0' ? 0 : 1) : -1;
  if (io_dtype != 1 || chunk < 32) return false;
  if (forced >= 0) return forced == 1;
  return (int64_t)n_seqs * h_v * (d / 64) >= kScanCUs;
}

// Fused workgroup shape: 0 for the wide one (every d_v column of a V head,
// so each chunk is prepared once per head), else the columns of a narrow
// block (16, 32 or 64) with separate output waves.  The wide block does the
// least work per chunk; GDN_FUSED_COLS=16, 32 or 64 forces a narrow width
// (tuning and comparison).
inline int fused_cols(const PrefillParams&, int d) {
  const char* e = std::getenv("GDN_FUSED_COLS");  // read per call: tests switch it in-process
  const int forced = e ? std::atoi(e) : 0;
  if ((forced == 16 || forced == 32 || forced == 64) && forced <= d) return forced;
  return 0;
}

template <int D, int C, int NC, int CT, bool W>
hipError_t launch_fused_cfg(const PrefillParams& p, const unsigned char* ws, hipStream_t stream) {
  using FL = FusedLayout<D, C, NC, CT, W>;
  static_assert(FL::bytes <= kLdsMax, "fused workgroup exceeds the LDS");
  const unsigned grid = scan_grid(p.n_seqs, p.h_qk, p.h_v, D / FL::cols);
  hipLaunchKernelGGL((fused_kernel<D, C, NC, CT, W>), dim3(grid), dim3(FL::threads), 0, stream, p, ws);
  return hipGetLastError();
}

template <int D, int C>
hipError_t launch_fused(const PrefillParams& p, hipStream_t stream) {
  unsigned char* ws = static_cast<unsigned char*>(p.workspace);
  if (p.cu_seqlens) {
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, stream, p.cu_seqlens, p.n_seqs, p.total_tokens, C,
                       p.emit_every, reinterpret_cast<int32_t*>(ws));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  switch (fused_cols(p, D)) {
    case 16: return launch_fused_cfg<D, C, 1, 1, false>(p, ws, stream);
    case 32: return launch_fused_cfg<D, C, 2, 1, false>(p, ws, stream);
    case 64: return launch_fused_cfg<D, C, 2, 2, false>(p, ws, stream);
    default: return launch_fused_cfg<D, C, D / 32, 2, true>(p, ws, stream);
  }
}

template <typename T, int D, int C>
hipError_t launch_t(const PrefillParams& p, hipStream_t stream) {
  if constexpr (fused_path<T, C>()) {
    if (use_fused(1, C, p.n_seqs, p.h_v, D)) return launch_fused<D, C>(p, stream);
  }
  if constexpr (!fits<T, D, C>()) {
    return hipErrorInvalidConfiguration;  // rejected by prefill_supported() first
  } else {
    constexpr int NW = kScanWaves, CT = kScanTiles;
    using SL = ScanLayout<T, D, C, NW, CT>;
    unsigned char* ws = static_cast<unsigned char*>(p.workspace);
    hipError_t e = hipSuccess;
    if (p.cu_seqlens) {  // one sequence needs no plan (PlanView)
      hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, stream, p.cu_seqlens, p.n_seqs, p.total_tokens, C,
                         p.emit_every, reinterpret_cast<int32_t*>(ws));
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const int grp = p.h_v / p.h_qk;
    const int vpw = sizeof(T) != 2 ? 1 : grp % 4 == 0 ? 4 : grp % 3 == 0 ? 3 : grp % 2 == 0 ? 2 : 1;
    if (p.total_tokens > 0) {
      const int64_t mc = max_chunks(p.total_tokens, p.n_seqs, C);
      e = vpw == 4 ? launch_prep<T, D, C, 4>(p, ws, mc, stream)
        : vpw == 3 ? launch_prep<T, D, C, 3>(p, ws, mc, stream)
        : vpw == 2 ? launch_prep<T, D, C, 2>(p, ws, mc, stream)
                   : launch_prep<T, D, C, 1>(p, ws, mc, stream);
      if (e != hipSuccess) return e;
    }
    if constexpr (sizeof(T) == 2) {
      const size_t recs_end = off_bytes(p.n_seqs) + (size_t)max_chunks(p.total_tokens, p.n_seqs, C) * p.h_v * Rec<T, C>::bytes;
      const SplitPlan sp = split_plan(1, p.total_tokens, p.n_seqs, p.h_v, D, C, p.emit_every, recs_end);
      ScanSplit ss{0, 0, nullptr, nullptr, nullptr, nullptr, nullptr};
      // 32- and 64-column workgroups: chain, output and mover waves
      constexpr unsigned narrow_threads = 64 * ((2 / kScan2Tiles) * (1 + kOutSplit<C>) + kMovers<C>);
      constexpr unsigned wide_threads = 64 * (4 / kScan2Tiles) * (1 + kOutSplit<C>);
      const auto narrow = scan2_kernel<D, C, kScan2Tiles, 2 / kScan2Tiles, kOutSplit<C>, kMovers<C>>;
      const auto wide = scan2_kernel<D, C, kScan2Tiles, 4 / kScan2Tiles, kOutSplit<C>, 0>;
      if (sp.on) {
        // one long sequence: two segments side by side
        float* st = reinterpret_cast<float*>(ws + sp.o_state);
        const size_t hs = (size_t)p.h_v * D * D;
        ss = ScanSplit{1, sp.m, st, st + hs, st + 2 * hs, reinterpret_cast<__bf16*>(ws + sp.o_w),
                       reinterpret_cast<__bf16*>(ws + sp.o_smb)};
        const unsigned grid = (unsigned)(3 * p.h_v * (D / sp.cols));
        hipLaunchKernelGGL(sp.cols == 32 ? narrow : wide, dim3(grid), dim3(sp.cols == 32 ? narrow_threads : wide_threads),
                           0, stream, p, static_cast<const unsigned char*>(ws), ss);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        const int ntile = (int)((p.total_tokens - sp.t_b + kJoinTok - 1) / kJoinTok);
        const int nstate = p.final_state ? p.h_v * (D / 16) : 0;
        hipLaunchKernelGGL(join_kernel<D>, dim3((unsigned)(nstate + ntile * p.h_v)), dim3(256), 0, stream, p, ss,
                           sp.t_b, nstate);
      } else if ((int64_t)p.n_seqs * p.h_v * (D / 32) <= kScanCUs) {
        // narrow workgroups when even they leave CUs idle
        const unsigned grid = scan_grid(p.n_seqs, p.h_qk, p.h_v, D / 32);
        hipLaunchKernelGGL(narrow, dim3(grid), dim3(narrow_threads), 0, stream, p,
                           static_cast<const unsigned char*>(ws), ss);
      } else {
        const unsigned grid = scan_grid(p.n_seqs, p.h_qk, p.h_v, D / 64);
        hipLaunchKernelGGL(wide, dim3(grid), dim3(wide_threads), 0, stream, p, static_cast<const unsigned char*>(ws), ss);
      }
    } else {
      const unsigned grid = scan_grid(p.n_seqs, p.h_qk, p.h_v, D / SL::cols);
      hipLaunchKernelGGL((scan_kernel<T, D, C, NW, CT>), dim3(grid), dim3(SL::threads), 0, stream, p,
                         static_cast<const unsigned char*>(ws));
    }
    return hipGetLastError();
  }
}

template <typename T, int D>
hipError_t launch_c(const PrefillParams& p, hipStream_t stream) {
  switch (p.chunk) {
    case 16: return launch_t<T, D, 16>(p, stream);
    case 32: return launch_t<T, D, 32>(p, stream);
    default: return launch_t<T, D, 64>(p, stream);
  }
}

template <typename T, int D>
bool fits_c(int chunk) {
  return chunk == 16 ? fits<T, D, 16>() : chunk == 32 ? fits<T, D, 32>() : fits<T, D, 64>();
}

template <typename T>
size_t rec_c(int chunk) {
  return chunk == 16 ? Rec<T, 16>::bytes : chunk == 32 ? Rec<T, 32>::bytes : Rec<T, 64>::bytes;
}

// ------------------------------------------------- calls without allocation
// The plan arrays of the fused kernel in a file-scope device array instead of
// a caller's workspace, for gdn_prefill_noalloc.  Each GPU the library runs
// on holds its own copy until the process ends.  In host code the array's
// name is a host-side stand-in, not a device address: its address on each
// device comes from hipGetSymbolAddress, taken once per device with that
// device current, and only that address reaches kernels.  Every call on a
// GPU shares its copy, so calls that overlap on one GPU race; the plan
// kernel writes every entry a call reads, so nothing needs clearing.
static __device__ __align__(256) unsigned char scratch[off_bytes(kNoAllocMaxSeqs)];

constexpr int kMaxDevices = 64;

hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = ptr;
  }
  *out = addr[dev];
  return hipSuccess;
}

}  // namespace

size_t prefill_workspace_bytes(int io_dtype, int64_t total_tokens, int n_seqs, int h_v, int d, int chunk,
                               int emit_every) {
  if (n_seqs < 1 || total_tokens < 0 || h_v < 1 || (chunk != 16 && chunk != 32 && chunk != 64)) return 0;
  if (use_fused(io_dtype, chunk, n_seqs, h_v, d)) return off_bytes(n_seqs);  // the fused kernel: the plan only
  const size_t rec = io_dtype == 1 ? rec_c<__bf16>(chunk) : rec_c<float>(chunk);
  const size_t recs_end = off_bytes(n_seqs) + (size_t)max_chunks(total_tokens, n_seqs, chunk) * h_v * rec;
  return split_plan(io_dtype, total_tokens, n_seqs, h_v, d, chunk, emit_every, recs_end).bytes;
}

bool prefill_supported(int io_dtype, int d, int chunk) {
  if (io_dtype == 1) return d == 128 ? fits_c<__bf16, 128>(chunk) : fits_c<__bf16, 64>(chunk);
  return d == 128 ? fits_c<float, 128>(chunk) : fits_c<float, 64>(chunk);
}

hipError_t launch_prefill(const PrefillParams& p, int io_dtype, int d, hipStream_t stream) {
  if (io_dtype == 1) return d == 128 ? launch_c<__bf16, 128>(p, stream) : launch_c<__bf16, 64>(p, stream);
  return d == 128 ? launch_c<float, 128>(p, stream) : launch_c<float, 64>(p, stream);
}

hipError_t launch_prefill_noalloc(const PrefillParams& p0, int d, hipStream_t stream) {
  PrefillParams p = p0;
  void* ptr = nullptr;
  const hipError_t e = scratch_address(&ptr);
  if (e != hipSuccess) return e;
  p.workspace = ptr;
  p.workspace_bytes = sizeof(scratch);
  if (d == 128) return p.chunk == 32 ? launch_fused<128, 32>(p, stream) : launch_fused<128, 64>(p, stream);
  return p.chunk == 32 ? launch_fused<64, 32>(p, stream) : launch_fused<64, 64>(p, stream);
}

}  // namespace gdn
