// GSA backward: gradients of the chunked forward with respect to q, k, v, the
// gate logits g and the initial slot states, given dO (and, optionally, the
// gradients of the final states).
//
// Method: "Gated Slot Attention for Efficient Linear-Time Sequence Modeling",
// Sec. 3.2-3.3 (the per-slot gated recurrence and its gate) and App. B (the
// training scheme: two GLA passes whose backward runs in reverse order, the
// gradient of the shared write intensity summed over both passes, and the
// forget-gate gradient formed from the products of each pass's inputs and
// outputs with their gradients by a reversed cumulative sum; states are
// recomputed rather than stored).
//
// Per unit (b, h), with alpha_t = sigmoid(g_t)^(1/tau), i_t = 1 - alpha_t,
// z_t = Kt q_t (pass-1 output), s_t = softmax(z_t) (or an element-wise read
// f(z_t), Table 2), o_t = Vt^T s_t:
//   ds_t = Vt dO_t,  dz_t = s_t * (ds_t - s_t . ds_t) (or f'(z_t) ds_t),
//   dq_t = Kt^T dz_t
//   adjoints (reverse in t): dVt = alpha_{t+1} dV_{t+1} + s_t dO_t^T,
//                            dKt = alpha_{t+1} dK_{t+1} + dz_t q_t^T
//   dk_t = dKt^T i_t,  dv_t = dVt^T i_t,  di_t = dKt k_t + dVt v_t
//   with G_t = sum_{r<=t} log alpha_r, the loss depends on G_t through
//   e^{G_t} on the reads of token t and e^{-G_t} on its writes, so
//   dL/dG_t = z_t dz_t + s_t ds_t - i_t di_t (+ the final-state term at T),
//   d log alpha_t = sum_{r>=t} dL/dG_r - alpha_t di_t,
//   dg_t = d log alpha_t * sigmoid(-g_t) / tau.
//
// Six launches, chunks of C = 64 tokens, one workgroup per (unit, chunk) for
// all but the scans:
//   1. bwd_map       chunk state maps (the state a chunk builds from zero, as
//                    a weighted sum over its tokens) and chunk decays, fp32;
//   2. bwd_scan<0>   chunk start states (forward scan of the maps);
//   3. bwd_walk_fwd  per chunk from its start state, token by token:
//                    z, s, ds, dz, dq, the reverse map of the chunk (what its
//                    reads add to the adjoint of its start state), and the
//                    per-token gate terms;
//   4. bwd_scan<1>   adjoints at chunk ends (reverse scan of the reverse maps
//                    from the final-state gradients); its carry out of chunk 0
//                    is the gradient of the initial states;
//   5. bwd_walk_rev  per chunk from its end adjoint, tokens in reverse: dk, dv
//                    and the chunk-local reversed sums of dL/dG;
//   6. bwd_gate      adds each chunk's carry (later chunks' sums and the
//                    final-state term) and applies the gate's derivative.
// The token walks keep both states (or both adjoints) of a unit in registers:
// thread (slot group sg, column group cg) of a 16 x 16 grid owns M/16 slot
// rows x D/16 columns of each, so that per-slot dot products are 16-lane row
// reductions inside a wave and per-column sums over slots run over the four
// slot groups of a wave and then, through LDS, over the four waves.  A unit's
// rows are placed by the sequence layout (a dense batch, or a packed batch of
// variable-length sequences; a unit has ceil(len / C) chunks, the workgroups
// of the grid's chunks past that return at once and the scans stop there).
#include <type_traits>

#include "../../include/gsa.h"
#include "bf16_common.hpp"
#include "common.hpp"
#include "internal.hpp"
#include "launch.hpp"

namespace gsa {
namespace bwd {

constexpr int C = 64;    // chunk length
constexpr int NT = 256;  // threads per workgroup: 4 waves, 16 x 16 thread grid

template <int DK, int DV, int M>
struct Shape {
  static constexpr int SPT = M / 16;  // slot rows per thread
  static constexpr int CK = DK / 16;  // key columns per thread
  static constexpr int CV = DV / 16;  // value columns per thread
  static constexpr int NE = M * (DK + DV);
  static_assert(M % 16 == 0 && DK % 64 == 0 && DV % 64 == 0, "shape");
};

// N consecutive elements (N = 2, 4 or 8; 4 N-byte aligned for bf16, 4 N for
// float) into fp32 registers
template <int N>
__device__ __forceinline__ void ldn(const float* p, float* o) {
  if constexpr (N == 2) {
    float2 x = *reinterpret_cast<const float2*>(p);
    o[0] = x.x; o[1] = x.y;
  } else {
#pragma unroll
    for (int j = 0; j < N; j += 4) {
      float4 x = *reinterpret_cast<const float4*>(p + j);
      o[j] = x.x; o[j + 1] = x.y; o[j + 2] = x.z; o[j + 3] = x.w;
    }
  }
}
template <int N>
__device__ __forceinline__ void ldn(const bf16_t* p, float* o) {
  if constexpr (N == 2) {
    uint32_t x = *reinterpret_cast<const uint32_t*>(p);
    o[0] = __uint_as_float(x << 16); o[1] = __uint_as_float(x & 0xffff0000u);
  } else if constexpr (N == 4) {
    uint2 x = *reinterpret_cast<const uint2*>(p);
    o[0] = __uint_as_float(x.x << 16); o[1] = __uint_as_float(x.x & 0xffff0000u);
    o[2] = __uint_as_float(x.y << 16); o[3] = __uint_as_float(x.y & 0xffff0000u);
  } else {
#pragma unroll
    for (int j = 0; j < N; j += 8) {
      uint4 x = *reinterpret_cast<const uint4*>(p + j);
      const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int e = 0; e < 4; e++) {
        o[j + 2 * e] = __uint_as_float(w[e] << 16);
        o[j + 2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
      }
    }
  }
}

template <int N>
__device__ __forceinline__ void stn(float* p, const float* v) {
  if constexpr (N == 2) {
    *reinterpret_cast<float2*>(p) = make_float2(v[0], v[1]);
  } else {
#pragma unroll
    for (int j = 0; j < N; j += 4) *reinterpret_cast<float4*>(p + j) = make_float4(v[j], v[j + 1], v[j + 2], v[j + 3]);
  }
}

// sum over the 16 lanes of a row (the column groups of one slot group) with
// DPP moves: quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror,
// row_mirror.  Every step adds a commuting pair, so all 16 lanes end with the
// same bits.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp_mov<0xB1>(x);
  x += dpp_mov<0x4E>(x);
  x += dpp_mov<0x141>(x);
  x += dpp_mov<0x140>(x);
  return x;
}

// sum / max over the four slot groups of a wave (lanes l, l ^ 16, l ^ 32,
// l ^ 48): gfx950's permlane swaps, no LDS round trip; every lane gets the
// same bits
__device__ __forceinline__ float sum_sg4(float x) { return bfk::group4_sum(x); }
__device__ __forceinline__ float max_sg4(float x) { return bfk::group4_max(x); }

struct Thread {
  int l, w, cg, sg;
  __device__ Thread() {
    l = threadIdx.x & 63;
    w = threadIdx.x >> 6;
    cg = l & 15;
    sg = w * 4 + (l >> 4);
  }
};

// Chunk inputs staged in LDS: rows t0 .. t1-1 of q, k (DK), v and dO (DV) in
// the I/O type, copied with 16-byte loads that are all in flight before the
// token loop (which then reads only LDS).
template <typename T, int DK, int DV, int M>
struct Stage {
  static constexpr int Q = 0, K = C * DK, V = 2 * C * DK, DO = 2 * C * DK + C * DV;
  static constexpr int elems = 2 * C * DK + 2 * C * DV;
  static constexpr unsigned bytes = elems * sizeof(T);
};

template <typename T>
__device__ __forceinline__ void copy_rows(T* __restrict__ dst, const T* __restrict__ src, int n_elems) {
  constexpr int V = 16 / sizeof(T);
  const uint4* s = reinterpret_cast<const uint4*>(src);
  uint4* d = reinterpret_cast<uint4*>(dst);
  for (int i = threadIdx.x; i < n_elems / V; i += blockDim.x) d[i] = s[i];
}

template <typename T, int DK, int DV, int M>
__device__ __forceinline__ void stage_chunk(T* lds, const T* qq, const T* kk, const T* vv, const T* dOo,
                                            size_t row0, int rows) {
  using SG = Stage<T, DK, DV, M>;
  copy_rows(lds + SG::Q, qq + row0 * DK, rows * DK);
  copy_rows(lds + SG::K, kk + row0 * DK, rows * DK);
  copy_rows(lds + SG::V, vv + row0 * DV, rows * DV);
  copy_rows(lds + SG::DO, dOo + row0 * DV, rows * DV);
}

// ------------------------------------------------------------ 1. maps
// The state chunk p builds from a zero start, and its decay prod alpha; also
// every token's alpha and write intensity 1 - alpha (fp32 [units, T, M] each),
// read by both token walks.  The map is the sum over the chunk's tokens j of
// Diag(prod_{r>j} alpha_r) i_j [k_j | v_j]^T: a product over the chunk with
// weights in [0, 1].  Thread (slot c, part) evaluates the gates of 16
// consecutive tokens of slot c, forms their suffix products, and the four
// parts of a slot combine their products through LDS; the product itself runs
// on the matrix cores in fp32 from the LDS-staged weights and k, v.
template <typename T, int DK, int DV, int M>
struct MapLds {
  static constexpr unsigned kv_bytes = C * (DK + DV) * sizeof(T);
  static constexpr unsigned bytes = kv_bytes + C * M * sizeof(float) + (NT / M) * M * sizeof(float);
};

template <typename T, int DK, int DV, int M, class Seq>
__global__ void __launch_bounds__(NT)
bwd_map(const T* __restrict__ kk, const T* __restrict__ vv, const T* __restrict__ gg,
        float* __restrict__ st, float* __restrict__ dec, float* __restrict__ al,
        float* __restrict__ wr, Seq seq, int P, float inv_tau) {
  using S = Shape<DK, DV, M>;
  constexpr int PARTS = NT / M, TPP = C / PARTS;  // parts per slot, tokens per part
  static_assert(NT % M == 0 && C % PARTS == 0, "gate split");
  extern __shared__ __align__(16) unsigned char lds_raw[];
  T* sk = reinterpret_cast<T*>(lds_raw);
  T* sv = sk + C * DK;
  float* sA = reinterpret_cast<float*>(lds_raw + C * (DK + DV) * sizeof(T));  // [C][M] weights
  float* ptot = sA + C * M;                                                     // [PARTS][M]
  const int p = blockIdx.y, u = blockIdx.x;
  const bfk::Span sp = seq.span(u);
  const int t0 = p * C, rows = min(sp.len, t0 + C) - t0;
  if (rows <= 0) return;  // past the sequence's end: no chunk (the scans stop before it)
  const size_t row0 = sp.base + t0;
  copy_rows(sk, kk + row0 * DK, rows * DK);
  copy_rows(sv, vv + row0 * DV, rows * DV);
  for (int i = rows * DK + threadIdx.x; i < C * DK; i += NT) sk[i] = Elem<T>::from_f(0.f);  // past the end
  for (int i = rows * DV + threadIdx.x; i < C * DV; i += NT) sv[i] = Elem<T>::from_f(0.f);
  {
    const int c = threadIdx.x % M, part = threadIdx.x / M, j0 = part * TPP;
    float av[TPP], wv[TPP];
#pragma unroll
    for (int x = 0; x < TPP; x++) {
      av[x] = 1.f;
      wv[x] = 0.f;
      if (j0 + x < rows) {
        const size_t e = (row0 + j0 + x) * M + c;
        gate_alpha_w(Elem<T>::to_f(gg[e]), inv_tau, av[x], wv[x]);
        al[e] = av[x];
        wr[e] = wv[x];
      }
    }
    float prod = 1.f;  // suffix product inside the part
#pragma unroll
    for (int x = TPP - 1; x >= 0; x--) {
      wv[x] *= prod;
      prod *= av[x];
    }
    ptot[part * M + c] = prod;
    __syncthreads();
    float after = 1.f;  // product of the later parts
    for (int q = part + 1; q < PARTS; q++) after *= ptot[q * M + c];
#pragma unroll
    for (int x = 0; x < TPP; x++) sA[(j0 + x) * M + c] = wv[x] * after;
    if (part == 0) dec[((size_t)u * P + p) * M + c] = prod * after;
  }
  __syncthreads();
  // the map A^T [k | v] on fp32 matrix cores (16x16x4 tiles, fp32 products):
  // A = sA [token][slot] is the transposed left operand, the staged k, v rows
  // the right one; the four waves share the (M/16) x ((DK+DV)/16) output tiles
  constexpr int NCOL = (DK + DV) / 16, TPW = (M / 16) * NCOL / 4;
  static_assert((M / 16) * NCOL % 4 == 0, "tiles per wave");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  f32x4 acc[TPW];
#pragma unroll
  for (int t = 0; t < TPW; t++) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int kend = (rows + 3) & ~3;
  for (int k0 = 0; k0 < kend; k0 += 4) {
    const int j = k0 + (lane >> 4);
#pragma unroll
    for (int t = 0; t < TPW; t++) {
      const int tile = wave * TPW + t, cb = tile / NCOL, nt = tile % NCOL;
      const float a = sA[j * M + 16 * cb + (lane & 15)];
      const int col = 16 * nt + (lane & 15);
      const float b = col < DK ? Elem<T>::to_f(sk[j * DK + col]) : Elem<T>::to_f(sv[j * DV + col - DK]);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[t], 0, 0, 0);
    }
  }
  float* base = st + ((size_t)u * P + p) * S::NE;
#pragma unroll
  for (int t = 0; t < TPW; t++) {
    const int tile = wave * TPW + t, cb = tile / NCOL, nt = tile % NCOL;
#pragma unroll
    for (int i = 0; i < 4; i++)
      base[(size_t)(16 * cb + 4 * (lane >> 4) + i) * (DK + DV) + 16 * nt + (lane & 15)] = acc[t][i];
  }
}

// ------------------------------------------------------------ 2./4. scans
// One thread per (unit, float4 of a slot row), serial over the chunks.
// REV = 0: slot p holds chunk p's map on entry and its start state on exit
// (W starts at the initial states ka / va, nullable = zero).
// REV = 1: slot p holds chunk p's reverse map on entry and, on exit, the
// adjoint of the state at chunk p's end from later tokens (W starts at the
// final-state gradients ka / va, nullable = zero); what is carried out of
// chunk 0 is written to kout / vout (nullable).
template <int DK, int DV, int M, int REV, class Seq>
__global__ void __launch_bounds__(256)
bwd_scan(float* __restrict__ ws, const float* __restrict__ dec, const float* __restrict__ ka,
         const float* __restrict__ va, float* __restrict__ kout, float* __restrict__ vout, Seq seq,
         int units, int P) {
  constexpr int NE = M * (DK + DV), BATCH = 8;
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long long)units * (NE / 4)) return;
  const int unit = (int)(gid / (NE / 4)), e = 4 * (int)(gid % (NE / 4));
  const int c = e / (DK + DV), cl = e % (DK + DV);
  const int Pu = (seq.span(unit).len + C - 1) / C;  // this unit's chunks (P for a dense batch)
  const size_t ko = ((size_t)unit * M + c) * DK + cl, vo = ((size_t)unit * M + c) * DV + cl - DK;
  f32x4 W = {0.f, 0.f, 0.f, 0.f};
  if (cl < DK) {
    if (ka) W = *reinterpret_cast<const f32x4*>(ka + ko);
  } else {
    if (va) W = *reinterpret_cast<const f32x4*>(va + vo);
  }
  f32x4* sl = reinterpret_cast<f32x4*>(ws + (size_t)unit * P * NE + e);
  const float* dc = dec + (size_t)unit * P * M + c;
  for (int n0 = 0; n0 < Pu; n0 += BATCH) {
    f32x4 x[BATCH];
    float d[BATCH];
#pragma unroll
    for (int i = 0; i < BATCH; i++) {
      if (n0 + i < Pu) {
        const int p = REV ? Pu - 1 - (n0 + i) : n0 + i;
        x[i] = sl[(size_t)p * (NE / 4)];
        d[i] = dc[(size_t)p * M];
      }
    }
#pragma unroll
    for (int i = 0; i < BATCH; i++) {
      if (n0 + i < Pu) {
        const int p = REV ? Pu - 1 - (n0 + i) : n0 + i;
        sl[(size_t)p * (NE / 4)] = W;
        W = d[i] * W + x[i];
      }
    }
  }
  if (REV) {
    if (cl < DK) {
      if (kout) *reinterpret_cast<f32x4*>(kout + ko) = W;
    } else {
      if (vout) *reinterpret_cast<f32x4*>(vout + vo) = W;
    }
  }
}

// ------------------------------------------------------------ 3. forward walk
// From chunk p's start state, token by token: the reads z, s, ds, dz, dq, the
// reverse map (sum over the chunk of e^{G_t} dz_t q_t^T and e^{G_t} s_t dO_t^T,
// G from the chunk start), and per token s, dz and z dz + s ds.  The chunk
// holding the last token also forms the final-state term dkf . K_T + dvf . V_T
// per slot (zero without final-state gradients).  ACT: the slot read, the
// softmax (dz = s (ds - s . ds)) or an element-wise f (s = f(z), dz = f'(z) ds).
template <typename T, int DK, int DV, int M, int ACT, class Seq>
__global__ void __launch_bounds__(NT)
bwd_walk_fwd(const T* __restrict__ qq, const T* __restrict__ kk, const T* __restrict__ vv,
             const float* __restrict__ al, const float* __restrict__ wr, const T* __restrict__ dOo,
             const float* __restrict__ st,
             const float* __restrict__ dkf, const float* __restrict__ dvf, T* __restrict__ dq,
             float* __restrict__ xu, float* __restrict__ sw, float* __restrict__ dzw,
             float* __restrict__ hw, float* __restrict__ fs, Seq seq, int P) {
  using S = Shape<DK, DV, M>;
  using SG = Stage<T, DK, DV, M>;
  extern __shared__ __align__(16) unsigned char lds_raw[];
  T* lds = reinterpret_cast<T*>(lds_raw);
  __shared__ float red[2][4][3];
  __shared__ float dqb[2][4][DK];
  const Thread th;
  const int p = blockIdx.y, u = blockIdx.x, c0 = th.sg * S::SPT;
  const bfk::Span sp = seq.span(u);
  const int t0 = p * C, t1 = min(sp.len, t0 + C);
  if (t1 <= t0) return;  // past the sequence's end: no chunk
  stage_chunk<T, DK, DV, M>(lds, qq, kk, vv, dOo, sp.base + t0, t1 - t0);
  float K[S::SPT][S::CK], V[S::SPT][S::CV], XK[S::SPT][S::CK], XV[S::SPT][S::CV], cum[S::SPT];
  {
    const float* base = st + ((size_t)u * P + p) * S::NE;
#pragma unroll
    for (int i = 0; i < S::SPT; i++) {
      const float* r = base + (size_t)(c0 + i) * (DK + DV);
      ldn<S::CK>(r + th.cg * S::CK, K[i]);
      ldn<S::CV>(r + DK + th.cg * S::CV, V[i]);
      cum[i] = 1.f;
#pragma unroll
      for (int j = 0; j < S::CK; j++) XK[i][j] = 0.f;
#pragma unroll
      for (int j = 0; j < S::CV; j++) XV[i][j] = 0.f;
    }
  }
  // this thread's slots' alpha and 1 - alpha, one token ahead
  float a_n[S::SPT], w_n[S::SPT];
  ldn<S::SPT>(al + (sp.base + t0) * M + c0, a_n);
  ldn<S::SPT>(wr + (sp.base + t0) * M + c0, w_n);
  __syncthreads();
  int n = 0;
  for (int t = t0; t < t1; t++, n++) {
    const int b = n & 1;
    const size_t row = sp.base + t;
    float av[S::SPT], wv[S::SPT], qv[S::CK], kv[S::CK], vv_[S::CV], dov[S::CV];
#pragma unroll
    for (int i = 0; i < S::SPT; i++) {
      av[i] = a_n[i];
      wv[i] = w_n[i];
    }
    if (t + 1 < t1) {
      ldn<S::SPT>(al + (row + 1) * M + c0, a_n);
      ldn<S::SPT>(wr + (row + 1) * M + c0, w_n);
    }
    ldn<S::CK>(lds + SG::Q + n * DK + th.cg * S::CK, qv);
    ldn<S::CK>(lds + SG::K + n * DK + th.cg * S::CK, kv);
    ldn<S::CV>(lds + SG::V + n * DV + th.cg * S::CV, vv_);
    ldn<S::CV>(lds + SG::DO + n * DV + th.cg * S::CV, dov);
    float z[S::SPT], ds[S::SPT];
#pragma unroll
    for (int i = 0; i < S::SPT; i++) {
      const float a = av[i], w = wv[i];
      cum[i] *= a;
      float zp = 0.f, dp = 0.f;
#pragma unroll
      for (int j = 0; j < S::CK; j++) {
        K[i][j] = a * K[i][j] + w * kv[j];
        zp += K[i][j] * qv[j];
      }
#pragma unroll
      for (int j = 0; j < S::CV; j++) {
        V[i][j] = a * V[i][j] + w * vv_[j];
        dp += V[i][j] * dov[j];
      }
      z[i] = row_sum16(zp);
      ds[i] = row_sum16(dp);
    }
    // softmax statistics of this wave's slots: max, sum of e^{z - max}, and
    // sum of e^{z - max} ds; then combined over the four waves (the barrier
    // also publishes the previous token's dq partial sums)
    if constexpr (ACT == kActSoftmax) {
      float mx = z[0];
#pragma unroll
      for (int i = 1; i < S::SPT; i++) mx = fmaxf(mx, z[i]);
      mx = max_sg4(mx);
      float se = 0.f, sd = 0.f;
#pragma unroll
      for (int i = 0; i < S::SPT; i++) {
        const float e = __expf(z[i] - mx);
        se += e;
        sd += e * ds[i];
      }
      se = sum_sg4(se);
      sd = sum_sg4(sd);
      if (th.l == 0) {
        red[b][th.w][0] = mx;
        red[b][th.w][1] = se;
        red[b][th.w][2] = sd;
      }
    }
    __syncthreads();
    if (n > 0 && threadIdx.x < DK) {  // dq of the previous token
      const float x = dqb[b ^ 1][0][threadIdx.x] + dqb[b ^ 1][1][threadIdx.x] + dqb[b ^ 1][2][threadIdx.x] +
                      dqb[b ^ 1][3][threadIdx.x];
      dq[(row - 1) * DK + threadIdx.x] = Elem<T>::from_f(x);
    }
    float s[S::SPT], dz[S::SPT];
    if constexpr (ACT == kActSoftmax) {
      float Mx = red[b][0][0];
#pragma unroll
      for (int x = 1; x < 4; x++) Mx = fmaxf(Mx, red[b][x][0]);
      float Se = 0.f, Sd = 0.f;
#pragma unroll
      for (int x = 0; x < 4; x++) {
        const float f = __expf(red[b][x][0] - Mx);
        Se += red[b][x][1] * f;
        Sd += red[b][x][2] * f;
      }
      const float inv = __builtin_amdgcn_rcpf(Se), dbar = Sd * inv;
#pragma unroll
      for (int i = 0; i < S::SPT; i++) {
        s[i] = __expf(z[i] - Mx) * inv;
        dz[i] = s[i] * (ds[i] - dbar);
      }
    } else {
#pragma unroll
      for (int i = 0; i < S::SPT; i++) {
        s[i] = slot_act<ACT>(z[i]);
        dz[i] = slot_act_grad<ACT>(z[i]) * ds[i];
      }
    }
    // dq partial sums over this wave's slots: all shuffles first, then one
    // store block (so that the cross-lane moves are in flight together)
    float dqp[S::CK];
#pragma unroll
    for (int j = 0; j < S::CK; j++) {
      float x = 0.f;
#pragma unroll
      for (int i = 0; i < S::SPT; i++) x += dz[i] * K[i][j];
      dqp[j] = x;
    }
#pragma unroll
    for (int j = 0; j < S::CK; j++) dqp[j] = sum_sg4(dqp[j]);
    if ((th.l >> 4) == 0) stn<S::CK>(&dqb[b][th.w][th.cg * S::CK], dqp);
    if (th.cg == 0) {
#pragma unroll
      for (int i = 0; i < S::SPT; i++) {
        sw[row * M + c0 + i] = s[i];
        dzw[row * M + c0 + i] = dz[i];
        hw[row * M + c0 + i] = z[i] * dz[i] + s[i] * ds[i];
      }
    }
#pragma unroll
    for (int i = 0; i < S::SPT; i++) {
      const float xs = cum[i] * dz[i], xv = cum[i] * s[i];
#pragma unroll
      for (int j = 0; j < S::CK; j++) XK[i][j] += xs * qv[j];
#pragma unroll
      for (int j = 0; j < S::CV; j++) XV[i][j] += xv * dov[j];
    }
  }
  __syncthreads();
  if (threadIdx.x < DK) {
    const int b = (n - 1) & 1;
    const float x = dqb[b][0][threadIdx.x] + dqb[b][1][threadIdx.x] + dqb[b][2][threadIdx.x] + dqb[b][3][threadIdx.x];
    dq[(sp.base + t1 - 1) * DK + threadIdx.x] = Elem<T>::from_f(x);
  }
  float* base = xu + ((size_t)u * P + p) * S::NE;
#pragma unroll
  for (int i = 0; i < S::SPT; i++) {
    float* r = base + (size_t)(c0 + i) * (DK + DV);
#pragma unroll
    for (int j = 0; j < S::CK; j += 4)
      *reinterpret_cast<f32x4*>(r + th.cg * S::CK + j) = f32x4{XK[i][j], XK[i][j + 1], XK[i][j + 2], XK[i][j + 3]};
#pragma unroll
    for (int j = 0; j < S::CV; j += 4)
      *reinterpret_cast<f32x4*>(r + DK + th.cg * S::CV + j) =
          f32x4{XV[i][j], XV[i][j + 1], XV[i][j + 2], XV[i][j + 3]};
  }
  if (t1 == sp.len) {  // the chunk holding the sequence's last token
#pragma unroll
    for (int i = 0; i < S::SPT; i++) {
      float x = 0.f;
      if (dkf) {
        float d[S::CK];
        ldn<S::CK>(dkf + ((size_t)u * M + c0 + i) * DK + th.cg * S::CK, d);
#pragma unroll
        for (int j = 0; j < S::CK; j++) x += d[j] * K[i][j];
      }
      if (dvf) {
        float d[S::CV];
        ldn<S::CV>(dvf + ((size_t)u * M + c0 + i) * DV + th.cg * S::CV, d);
#pragma unroll
        for (int j = 0; j < S::CV; j++) x += d[j] * V[i][j];
      }
      x = row_sum16(x);
      if (th.cg == 0) fs[(size_t)u * M + c0 + i] = x;
    }
  }
}

// ------------------------------------------------------------ 5. reverse walk
// From the adjoint at chunk p's end, tokens in reverse: dk, dv, and per token
// the chunk-local reversed sum of dL/dG minus alpha di (written over z dz +
// s ds); the chunk's total goes to tot.
template <typename T, int DK, int DV, int M, class Seq>
__global__ void __launch_bounds__(NT)
bwd_walk_rev(const T* __restrict__ qq, const T* __restrict__ kk, const T* __restrict__ vv,
             const float* __restrict__ al, const float* __restrict__ wr, const T* __restrict__ dOo,
             const float* __restrict__ xu,
             const float* __restrict__ sw, const float* __restrict__ dzw, float* __restrict__ hw,
             float* __restrict__ tot, T* __restrict__ dk, T* __restrict__ dv, Seq seq, int P) {
  using S = Shape<DK, DV, M>;
  using SG = Stage<T, DK, DV, M>;
  extern __shared__ __align__(16) unsigned char lds_raw[];
  T* lds = reinterpret_cast<T*>(lds_raw);
  __shared__ float kvb[2][4][DK + DV];
  const Thread th;
  const int p = blockIdx.y, u = blockIdx.x, c0 = th.sg * S::SPT;
  const bfk::Span sp = seq.span(u);
  const int t0 = p * C, t1 = min(sp.len, t0 + C);
  if (t1 <= t0) return;  // past the sequence's end: no chunk
  stage_chunk<T, DK, DV, M>(lds, qq, kk, vv, dOo, sp.base + t0, t1 - t0);
  float AK[S::SPT][S::CK], AV[S::SPT][S::CV], R[S::SPT];
  {
    const float* base = xu + ((size_t)u * P + p) * S::NE;
#pragma unroll
    for (int i = 0; i < S::SPT; i++) {
      const float* r = base + (size_t)(c0 + i) * (DK + DV);
      ldn<S::CK>(r + th.cg * S::CK, AK[i]);
      ldn<S::CV>(r + DK + th.cg * S::CV, AV[i]);
      R[i] = 0.f;
    }
  }
  // per-token s, dz, z dz + s ds, alpha and 1 - alpha of this thread's slots,
  // one token ahead
  float sv_n[S::SPT], dzv_n[S::SPT], hv_n[S::SPT], a_n[S::SPT], w_n[S::SPT];
  {
    const size_t r = sp.base + t1 - 1;
    ldn<S::SPT>(sw + r * M + c0, sv_n);
    ldn<S::SPT>(dzw + r * M + c0, dzv_n);
    ldn<S::SPT>(hw + r * M + c0, hv_n);
    ldn<S::SPT>(al + r * M + c0, a_n);
    ldn<S::SPT>(wr + r * M + c0, w_n);
  }
  __syncthreads();
  int n = 0;
  for (int t = t1 - 1; t >= t0; t--, n++) {
    const int b = n & 1, lt = t - t0;
    const size_t row = sp.base + t;
    float sv[S::SPT], dzv[S::SPT], hv[S::SPT], a[S::SPT], w[S::SPT], di[S::SPT];
    float qv[S::CK], kv[S::CK], vv_[S::CV], dov[S::CV];
#pragma unroll
    for (int i = 0; i < S::SPT; i++) {
      sv[i] = sv_n[i];
      dzv[i] = dzv_n[i];
      hv[i] = hv_n[i];
      a[i] = a_n[i];
      w[i] = w_n[i];
    }
    if (t > t0) {
      ldn<S::SPT>(sw + (row - 1) * M + c0, sv_n);
      ldn<S::SPT>(dzw + (row - 1) * M + c0, dzv_n);
      ldn<S::SPT>(hw + (row - 1) * M + c0, hv_n);
      ldn<S::SPT>(al + (row - 1) * M + c0, a_n);
      ldn<S::SPT>(wr + (row - 1) * M + c0, w_n);
    }
    ldn<S::CK>(lds + SG::Q + lt * DK + th.cg * S::CK, qv);
    ldn<S::CK>(lds + SG::K + lt * DK + th.cg * S::CK, kv);
    ldn<S::CV>(lds + SG::V + lt * DV + th.cg * S::CV, vv_);
    ldn<S::CV>(lds + SG::DO + lt * DV + th.cg * S::CV, dov);
#pragma unroll
    for (int i = 0; i < S::SPT; i++) {
      float pk = 0.f, pv = 0.f;
#pragma unroll
      for (int j = 0; j < S::CK; j++) {
        AK[i][j] += dzv[i] * qv[j];
        pk += AK[i][j] * kv[j];
      }
#pragma unroll
      for (int j = 0; j < S::CV; j++) {
        AV[i][j] += sv[i] * dov[j];
        pv += AV[i][j] * vv_[j];
      }
      di[i] = row_sum16(pk) + row_sum16(pv);
    }
    // dk, dv partial sums over this wave's slots: all shuffles first, then
    // one store block
    float pk_[S::CK], pv_[S::CV];
#pragma unroll
    for (int j = 0; j < S::CK; j++) {
      float x = 0.f;
#pragma unroll
      for (int i = 0; i < S::SPT; i++) x += w[i] * AK[i][j];
      pk_[j] = x;
    }
#pragma unroll
    for (int j = 0; j < S::CV; j++) {
      float x = 0.f;
#pragma unroll
      for (int i = 0; i < S::SPT; i++) x += w[i] * AV[i][j];
      pv_[j] = x;
    }
#pragma unroll
    for (int j = 0; j < S::CK; j++) pk_[j] = sum_sg4(pk_[j]);
#pragma unroll
    for (int j = 0; j < S::CV; j++) pv_[j] = sum_sg4(pv_[j]);
    if ((th.l >> 4) == 0) {
      stn<S::CK>(&kvb[b][th.w][th.cg * S::CK], pk_);
      stn<S::CV>(&kvb[b][th.w][DK + th.cg * S::CV], pv_);
    }
#pragma unroll
    for (int i = 0; i < S::SPT; i++) {
#pragma unroll
      for (int j = 0; j < S::CK; j++) AK[i][j] *= a[i];
#pragma unroll
      for (int j = 0; j < S::CV; j++) AV[i][j] *= a[i];
      R[i] += hv[i] - w[i] * di[i];
    }
    if (th.cg == 0) {
#pragma unroll
      for (int i = 0; i < S::SPT; i++) hw[row * M + c0 + i] = R[i] - a[i] * di[i];
    }
    __syncthreads();
    for (int e = threadIdx.x; e < DK + DV; e += NT) {
      const float x = kvb[b][0][e] + kvb[b][1][e] + kvb[b][2][e] + kvb[b][3][e];
      if (e < DK) dk[row * DK + e] = Elem<T>::from_f(x);
      else dv[row * DV + e - DK] = Elem<T>::from_f(x);
    }
  }
  if (th.cg == 0) {
#pragma unroll
    for (int i = 0; i < S::SPT; i++) tot[((size_t)u * P + p) * M + c0 + i] = R[i];
  }
}

// ------------------------------------------------------------ 6. gate
// dg = (chunk-local reversed sum + carry) * sigmoid(-g) / tau, the carry of
// chunk p being the final-state term plus the totals of chunks p+1 .. P-1.
template <typename T, int M, class Seq>
__global__ void __launch_bounds__(256)
bwd_gate(const T* __restrict__ gg, const float* __restrict__ hw, const float* __restrict__ tot,
         const float* __restrict__ fs, T* __restrict__ dg, Seq seq, int P, float inv_tau) {
  __shared__ float carry[M];
  const int p = blockIdx.y, u = blockIdx.x;
  const bfk::Span sp = seq.span(u);
  const int t0 = p * C, Pu = (sp.len + C - 1) / C;
  if (p >= Pu) return;  // past the sequence's end: no chunk
  if (threadIdx.x < M) {
    float c = fs[(size_t)u * M + threadIdx.x];
    const float* tp = tot + (size_t)u * P * M + threadIdx.x;
#pragma unroll 8
    for (int x = p + 1; x < Pu; x++) c += tp[(size_t)x * M];
    carry[threadIdx.x] = c;
  }
  __syncthreads();
  const int n = min(C, sp.len - t0) * M;
  const size_t base = (sp.base + t0) * M;
  for (int e = threadIdx.x; e < n; e += 256) {
    const int c = e % M;
    const float gv = Elem<T>::to_f(gg[base + e]);
    const float sneg = 1.f / (1.f + __expf(gv));  // sigmoid(-g): 0 at +inf, 1 at -inf
    dg[base + e] = Elem<T>::from_f((hw[base + e] + carry[c]) * sneg * inv_tau);
  }
}

// ------------------------------------------------------------ host side
struct Ws {
  float *st, *xu, *dec, *sw, *dzw, *hw, *al, *wr, *tot, *fs;
};

// floats of workspace for U units of P chunks each (one launch sequence) over
// `rows` token rows in all (the per-token arrays are indexed by token row)
inline size_t ws_floats(size_t U, size_t P, size_t rows, int dk, int dv, int m) {
  return 2 * U * P * (size_t)m * (dk + dv) + 2 * U * P * m + 5 * rows * m + U * m;
}

inline Ws carve(float* w, size_t U, size_t P, size_t rows, int dk, int dv, int m) {
  const size_t NE = (size_t)m * (dk + dv);
  Ws s;
  s.st = w;
  s.xu = s.st + U * P * NE;
  s.dec = s.xu + U * P * NE;
  s.tot = s.dec + U * P * m;
  s.sw = s.tot + U * P * m;
  s.dzw = s.sw + rows * m;
  s.hw = s.dzw + rows * m;
  s.al = s.hw + rows * m;
  s.wr = s.al + rows * m;
  s.fs = s.wr + rows * m;
  return s;
}

// One launch sequence over U units of P chunks each, the units' rows placed by
// seq; k0 .. dv0 point at these units' states.
template <typename T, int DK, int DV, int M, int ACT, class Seq>
void launch_seq(const GsaBwdLaunch& a, const Seq& seq, int U, int P, const Ws& w, const float* k0,
                const float* v0, const float* dkf, const float* dvf, float* dk0, float* dv0,
                void* const* events) {
  const float inv_tau = 1.0f / a.tau;
  const T *q = (const T*)a.q, *k = (const T*)a.k, *v = (const T*)a.v, *g = (const T*)a.g,
          *dO = (const T*)a.d_o;
  hipStream_t s = (hipStream_t)a.stream;
  using SG = Stage<T, DK, DV, M>;
  static const bool lds_set = [] {  // once per instantiation and process
    (void)hipFuncSetAttribute((const void*)bwd_map<T, DK, DV, M, Seq>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, MapLds<T, DK, DV, M>::bytes);
    (void)hipFuncSetAttribute((const void*)bwd_walk_fwd<T, DK, DV, M, ACT, Seq>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, SG::bytes);
    (void)hipFuncSetAttribute((const void*)bwd_walk_rev<T, DK, DV, M, Seq>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, SG::bytes);
    return true;
  }();
  (void)lds_set;
  // units along x: consecutive workgroups (which the dispatcher deals round
  // robin to the eight XCDs) are different units' chunk p, so every XCD gets
  // an even share of every chunk index (with chunks along x, chunk p of every
  // unit would land on XCD p mod 8, and a packed batch's late chunks, which
  // only long sequences have, on a few XCDs)
  const dim3 grid(U, P);
  const long long ne = (long long)U * M * (DK + DV) / 4;
  const dim3 sgrid((unsigned)((ne + 255) / 256));
  constexpr unsigned map_lds = MapLds<T, DK, DV, M>::bytes;
  hipLaunchKernelGGL((bwd_map<T, DK, DV, M, Seq>), grid, dim3(NT), map_lds, s, k, v, g, w.st, w.dec, w.al, w.wr,
                     seq, P, inv_tau);
  hipLaunchKernelGGL((bwd_scan<DK, DV, M, 0, Seq>), sgrid, dim3(256), 0, s, w.st, (const float*)w.dec, k0, v0,
                     (float*)nullptr, (float*)nullptr, seq, U, P);
  launch_timed(bwd_walk_fwd<T, DK, DV, M, ACT, Seq>, grid, dim3(NT), SG::bytes, a.stream, events, 0, 1, q, k,
               v, (const float*)w.al, (const float*)w.wr, dO, (const float*)w.st, dkf, dvf, (T*)a.dq, w.xu,
               w.sw, w.dzw, w.hw, w.fs, seq, P);
  hipLaunchKernelGGL((bwd_scan<DK, DV, M, 1, Seq>), sgrid, dim3(256), 0, s, w.xu, (const float*)w.dec, dkf, dvf,
                     dk0, dv0, seq, U, P);
  launch_timed(bwd_walk_rev<T, DK, DV, M, Seq>, grid, dim3(NT), SG::bytes, a.stream, events, 2, 3, q, k, v,
               (const float*)w.al, (const float*)w.wr, dO, (const float*)w.xu, (const float*)w.sw,
               (const float*)w.dzw, w.hw, w.tot, (T*)a.dk, (T*)a.dv, seq, P);
  hipLaunchKernelGGL((bwd_gate<T, M, Seq>), grid, dim3(256), 0, s, g, (const float*)w.hw, (const float*)w.tot,
                     (const float*)w.fs, (T*)a.dg, seq, P, inv_tau);
}

template <typename T, int DK, int DV, int M, int ACT>
int launch(const GsaBwdLaunch& a) {
  const size_t MK = (size_t)a.H * M * DK, MV = (size_t)a.H * M * DV;  // states per batch entry
  if (!a.cu_seqlens) {
    const int U = a.B * a.H, P = (a.T + C - 1) / C;
    if (a.T == 0) {  // no tokens: the initial states' gradients are the final ones'
      state_copy(a.dk0, a.dkf, (size_t)a.B * MK, a.stream);
      state_copy(a.dv0, a.dvf, (size_t)a.B * MV, a.stream);
      for (int e = 0; e < 4; e++) record_event(a.events, e, a.stream);
      return 0;
    }
    if constexpr (std::is_same<T, bf16_t>::value && ACT != kActRelu)  // the chunk form on the matrix cores
      return gsa_bwd_bf16_dispatch(DK, DV, M, &a, false, (size_t)U, a.T) == 0 ? 0 : -1;
    const Ws w = carve(a.ws, U, P, (size_t)U * a.T, DK, DV, M);
    launch_seq<T, DK, DV, M, ACT>(a, bfk::DenseSeqs{a.T}, U, P, w, a.k0, a.v0, a.dkf, a.dvf, a.dk0, a.dv0,
                                  a.events);
    return 0;
  }
  // A packed batch of variable-length sequences: groups of at most
  // kMaxVarSeqs sequences, one launch sequence each (a group's offsets travel
  // in the kernel arguments), one after the other on the stream.  They share
  // the workspace: its chunk arrays are sized for the largest group and the
  // longest sequence, its per-token arrays cover every packed row.
  const int n = a.n_seqs, total = a.cu_seqlens[n];
  int tmax = 0;
  for (int i = 0; i < n; i++) tmax = max(tmax, a.cu_seqlens[i + 1] - a.cu_seqlens[i]);
  const Ws w = carve(a.ws, (size_t)min(n, kMaxVarSeqs) * a.H, (tmax + C - 1) / C, (size_t)a.H * total, DK, DV, M);
  const int groups = (n + kMaxVarSeqs - 1) / kMaxVarSeqs;
  if (groups > 1) {
    record_event(a.events, 0, a.stream);
    record_event(a.events, 1, a.stream);
  }
  for (int g0 = 0; g0 < n; g0 += kMaxVarSeqs) {
    const int ng = min(kMaxVarSeqs, n - g0);
    bfk::VarSeqs vs{};
    vs.H = a.H;
    vs.total = total;
    int tg = 0;
    for (int i = 0; i <= ng; i++) vs.cu[i] = a.cu_seqlens[g0 + i];
    for (int i = 0; i < ng; i++) {
      vs.order[i] = i;
      tg = max(tg, vs.cu[i + 1] - vs.cu[i]);
    }
    const float* k0 = a.k0 ? a.k0 + g0 * MK : nullptr;
    const float* v0 = a.v0 ? a.v0 + g0 * MV : nullptr;
    const float* dkf = a.dkf ? a.dkf + g0 * MK : nullptr;
    const float* dvf = a.dvf ? a.dvf + g0 * MV : nullptr;
    float* dk0 = a.dk0 ? a.dk0 + g0 * MK : nullptr;
    float* dv0 = a.dv0 ? a.dv0 + g0 * MV : nullptr;
    if (tg == 0) {  // only empty sequences
      state_copy(dk0, dkf, (size_t)ng * MK, a.stream);
      state_copy(dv0, dvf, (size_t)ng * MV, a.stream);
      if (groups == 1)  // the call's only group: its events still stamp the (empty) work
        for (int e = 0; e < 4; e++) record_event(a.events, e, a.stream);
      continue;
    }
    launch_seq<T, DK, DV, M, ACT>(a, vs, ng * a.H, (tg + C - 1) / C, w, k0, v0, dkf, dvf, dk0, dv0,
                                  groups == 1 ? a.events : nullptr);
  }
  if (groups > 1) {
    record_event(a.events, 2, a.stream);
    record_event(a.events, 3, a.stream);
  }
  return 0;
}

template <typename T, int DK, int DV, int M>
int launch_act(const GsaBwdLaunch& a) {
  switch (a.act) {
    case kActSoftmax: return launch<T, DK, DV, M, kActSoftmax>(a);
    case kActIdentity: return launch<T, DK, DV, M, kActIdentity>(a);
    case kActSwish: return launch<T, DK, DV, M, kActSwish>(a);
    case kActRelu: return launch<T, DK, DV, M, kActRelu>(a);
    case kActRelu2: return launch<T, DK, DV, M, kActRelu2>(a);
    default: return -1;
  }
}

}  // namespace bwd

size_t gsa_bwd_ws_bytes(size_t units, size_t chunks, size_t rows, int dk, int dv, int m) {
  return bwd::ws_floats(units, chunks, rows, dk, dv, m) * sizeof(float);
}

size_t gsa_bwd_need_bytes(int dtype, int act, bool packed, size_t units, size_t chunks, size_t rows, int T,
                          int dk, int dv, int m) {
  if (gsa_bwd_on_mfma(dtype, act, packed)) {
    const long long b = gsa_bwd_bf16_dispatch(dk, dv, m, nullptr, true, units, T);
    if (b >= 0) return (size_t)b;
  }
  return gsa_bwd_ws_bytes(units, chunks, rows, dk, dv, m);
}

#define GSA_BWD_CASE(TY, DT, DK_, DV_, M_)                                    \
  if (dtype == DT && dk == DK_ && dv == DV_ && m == M_)                       \
    return query ? 0 : bwd::launch_act<TY, DK_, DV_, M_>(*a);

int gsa_bwd_dispatch(int dtype, int dk, int dv, int m, const GsaBwdLaunch* a, bool query) {
  // 128 slots: bf16 dense batches on the matrix cores as two slot groups (not
  // the ReLU read, not packed batches: the caller rejects those)
  if (slot_groups(dtype, m) == 2 && dk == dv && (dk == 128 || dk == 64)) {
    if (query) return 0;
    if (a->cu_seqlens || a->act == kActRelu) return -1;
    if (a->T == 0) {
      const size_t MK = (size_t)a->H * m * dk, MV = (size_t)a->H * m * dv;
      state_copy(a->dk0, a->dkf, (size_t)a->B * MK, a->stream);
      state_copy(a->dv0, a->dvf, (size_t)a->B * MV, a->stream);
      for (int e = 0; e < 4; e++) record_event(a->events, e, a->stream);
      return 0;
    }
    return gsa_bwd_bf16_dispatch(dk, dv, m, a, false, (size_t)a->B * a->H, a->T) == 0 ? 0 : -1;
  }
  GSA_BWD_CASE(bf16_t, 1, 128, 128, 64)
  GSA_BWD_CASE(bf16_t, 1, 64, 64, 32)
  GSA_BWD_CASE(bf16_t, 1, 128, 128, 32)
  GSA_BWD_CASE(bf16_t, 1, 64, 64, 64)
  GSA_BWD_CASE(float, 0, 128, 128, 64)
  GSA_BWD_CASE(float, 0, 64, 64, 32)
  GSA_BWD_CASE(float, 0, 128, 128, 32)
  GSA_BWD_CASE(float, 0, 64, 64, 64)
  return -1;
}

}  // namespace gsa
