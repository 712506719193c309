// Chunkwise GSA forward on gfx950.
//
// Method: "Gated Slot Attention for Efficient Linear-Time Sequence Modeling"
// (arXiv 2409.07146).  Per (batch, head) unit, with m slots and
// alpha_t = sigmoid(g_t)^(1/tau) (Sec. 3.3):
//   Kt_t = Diag(alpha_t) Kt_{t-1} + (1 - alpha_t) k_t^T     (pass-1 state)
//   s_t  = softmax over slots of Kt_t q_t                   (Sec. 3.2 / App. B)
//   Vt_t = Diag(alpha_t) Vt_{t-1} + (1 - alpha_t) v_t^T     (pass-2 state)
//   o_t  = Vt_t^T s_t
// The chunk form (App. A.1, App. B) splits each chunk's outputs into a read of
// the chunk-start state plus an intra-chunk causal term, both as matrix-core
// contractions.  Both states decay and write with the same gates and do not
// depend on q or s, so they are carried together as one fp32 state
// W = [Kt | Vt] in R^{m x (dk+dv)}.
//
// Three launches (no inter-workgroup waiting anywhere):
//   A  gsa_seg_state : per (unit, segment of S chunks), the segment's affine
//                      state map W -> Diag(a) W + D from a zero start.
//   B  gsa_seg_scan  : per unit, serial over segments, elementwise fp32:
//                      start state of every segment (+ the final state).
//   C  gsa_seg_out   : per (unit, segment), from its start state, the chunks'
//                      outputs, carrying W chunk to chunk in MFMA accumulators.
// With one segment per unit, A and B are skipped.
//
// Inside a chunk (C = 64 tokens), with E_j = prod_{i<=j} alpha_i per slot and
// S_r = prod_{i>r} alpha_i, the decay between tokens r <= j is E_j / E_r.  When
// every slot's whole-chunk product is >= e^-40 the factorisation
// (w_r / E_r) * E_j is formed directly (fast path, all MFMA).  Otherwise the
// chunk is run as the exact token recurrence on the register-resident state
// (slow path), which needs no division by a decay product at all.
#include "common.hpp"
#include "internal.hpp"
#include "launch.hpp"

namespace gsa {

constexpr int kC = 64;    // chunk length handled by the kernels
constexpr int kNW = 8;    // waves per workgroup
constexpr int kNT = kNW * 64;

template <typename T, int DK, int DV, int M>
struct GsaLds {
  static constexpr int PAD = Pad<T>::v;
  static constexpr int LDK = DK + PAD, LDV = DV + PAD, LDM = M + PAD, LDC = kC + PAD;
  static constexpr int LDW = DK + DV + PAD, LDE = M + 4;
  static constexpr int TS = (int)sizeof(T);
  static constexpr int oQ = 0;
  static constexpr int oK = oQ + kC * LDK * TS;
  static constexpr int oV = oK + kC * LDK * TS;
  static constexpr int oW = oV + kC * LDV * TS;
  static constexpr int oU = oW + M * LDW * TS;
  // fast-path factors
  static constexpr int oE = oU;
  static constexpr int oX = oE + kC * LDE * 4;
  static constexpr int oZ = oX + kC * LDM * TS;
  static constexpr int oSE = oZ + kC * LDM * TS;
  static constexpr int szFast = kC * LDE * 4 + 3 * kC * LDM * TS;
  // slow-path per-token gates
  static constexpr int oAl = oU;
  static constexpr int oWr = oU + kC * M * 4;
  static constexpr int szSlow = 2 * kC * M * 4;
  static constexpr int szU = szFast > szSlow ? szFast : szSlow;
  static constexpr int oA = oU + szU;
  static constexpr int oRed = oA + kC * LDC * TS;          // 2 x [C][M/16] fp32
  static constexpr int oDec = oRed + 2 * kC * (M / 16) * 4;  // [M] fp32
  static constexpr int oZp = oDec + M * 4;                 // [DK/16][M] fp32
  static constexpr int oOp = oZp + (DK / 16) * M * 4;      // [M/16][DV] fp32
  static constexpr int oS = oOp + (M / 16) * DV * 4;       // [M] fp32
  static constexpr int total = oS + M * 4;
  static_assert(oK % 16 == 0 && oV % 16 == 0 && oW % 16 == 0 && oU % 16 == 0 && oX % 16 == 0 &&
                    oZ % 16 == 0 && oSE % 16 == 0 && oA % 16 == 0 && oRed % 16 == 0,
                "LDS tiles must stay 16-byte aligned");
};

template <typename T, int DK, int DV, int M>
struct GsaStateLds {
  static constexpr int PAD = Pad<T>::v;
  static constexpr int LDK = DK + PAD, LDV = DV + PAD, LDM = M + PAD;
  static constexpr int TS = (int)sizeof(T);
  static constexpr int oK = 0;
  static constexpr int oV = oK + kC * LDK * TS;
  static constexpr int oZ = oV + kC * LDV * TS;
  static constexpr int oDec = oZ + kC * LDM * TS;
  static constexpr int total = oDec + M * 4;
};

// ---------------------------------------------------------------- tile loads
// A [C][D] row-major chunk tile of T, moved as 16-byte vectors, 512 threads.
template <typename T, int D>
struct TileIO {
  static constexpr int VPR = D * (int)sizeof(T) / 16;  // vectors per row
  static constexpr int NV = kC * VPR / kNT;            // vectors per thread
  static_assert(NV >= 1 && (kC * VPR) % kNT == 0, "tile/thread mismatch");
  static constexpr int EPV = 16 / (int)sizeof(T);
  uint4 r[NV];
  __device__ __forceinline__ void load(const T* __restrict__ base, int rows_valid, int tid) {
#pragma unroll
    for (int i = 0; i < NV; i++) {
      int idx = tid + kNT * i;
      int row = idx / VPR, cv = idx % VPR;
      if (row < rows_valid)
        r[i] = *reinterpret_cast<const uint4*>(base + (size_t)row * D + cv * EPV);
      else
        r[i] = make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store_lds(T* dst, int ld, int tid) const {
#pragma unroll
    for (int i = 0; i < NV; i++) {
      int idx = tid + kNT * i;
      int row = idx / VPR, cv = idx % VPR;
      *reinterpret_cast<uint4*>(dst + row * ld + cv * EPV) = r[i];
    }
  }
};

// SPT consecutive values of one row (gate logits in the gate-prep mapping).
template <typename T, int N>
struct RowVec {
  float v[N];
  __device__ __forceinline__ void load(const T* __restrict__ p, bool valid) {
    if (!valid) {
#pragma unroll
      for (int s = 0; s < N; s++) v[s] = 0.f;
      return;
    }
    constexpr int BYTES = N * (int)sizeof(T);
    if constexpr (BYTES % 16 == 0) {
      constexpr int NV = BYTES / 16, EPV = 16 / (int)sizeof(T);
#pragma unroll
      for (int i = 0; i < NV; i++) {
        uint4 u = *reinterpret_cast<const uint4*>(p + i * EPV);
        const T* e = reinterpret_cast<const T*>(&u);
#pragma unroll
        for (int s = 0; s < EPV; s++) v[i * EPV + s] = Elem<T>::to_f(e[s]);
      }
    } else if constexpr (BYTES == 8) {
      uint2 u = *reinterpret_cast<const uint2*>(p);
      const T* e = reinterpret_cast<const T*>(&u);
#pragma unroll
      for (int s = 0; s < N; s++) v[s] = Elem<T>::to_f(e[s]);
    } else {
#pragma unroll
      for (int s = 0; s < N; s++) v[s] = Elem<T>::to_f(p[s]);
    }
  }
};

// ------------------------------------------------------------- gate prep
// Wave w owns slots [w*SPT, (w+1)*SPT); lane j owns chunk row j.  Computes per
// (j, c): alpha, 1-alpha, E_j = prod_{i<=j} alpha_i, S_j = prod_{i>j} alpha_i,
// via wave-wide multiplicative scans.  Padding rows (j >= valid) are no-ops
// (alpha = 1, write 0).
template <int SPT>
struct Gates {
  float a[SPT], w[SPT], E[SPT], Sx[SPT];
  __device__ __forceinline__ void compute(const float* g, bool valid, float inv_tau, int lane) {
#pragma unroll
    for (int s = 0; s < SPT; s++) {
      if (valid) {
        gate_alpha_w(g[s], inv_tau, a[s], w[s]);
      } else {
        a[s] = 1.f;
        w[s] = 0.f;
      }
      E[s] = a[s];
      Sx[s] = a[s];
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
#pragma unroll
      for (int s = 0; s < SPT; s++) {
        float up = __shfl_up(E[s], off, 64);
        float dn = __shfl_down(Sx[s], off, 64);
        if (lane >= off) E[s] *= up;
        if (lane + off < 64) Sx[s] *= dn;
      }
    }
    // Sx is now the inclusive suffix product; shift to exclusive
#pragma unroll
    for (int s = 0; s < SPT; s++) {
      float nx = __shfl_down(Sx[s], 1, 64);
      Sx[s] = (lane == 63) ? 1.f : nx;
    }
  }
};

// ------------------------------------------------------ phase A: state map
// grid (nseg_state, units).  Writes the segment's state map from a zero start:
// D = sum over its tokens of Diag(prod_{i>r} alpha_i) (1-alpha_r) [k_r|v_r]^T,
// and the segment decay product a = prod alpha_i.
template <typename T, int DK, int DV, int M>
__global__ void __launch_bounds__(kNT, 1)
gsa_seg_state(const T* __restrict__ kk, const T* __restrict__ vv, const T* __restrict__ gg,
              float* __restrict__ ws_state, float* __restrict__ ws_dec, int T_len, int S, int P,
              float inv_tau) {
  using L = GsaStateLds<T, DK, DV, M>;
  using O = Op<T>;
  constexpr int SPT = M / kNW;
  constexpr int NCT = (DK + DV) / 16;
  constexpr int NTS = (M / 16) * NCT;
  constexpr int TPW = (NTS + kNW - 1) / kNW;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  T* sK = reinterpret_cast<T*>(smem + L::oK);
  T* sV = reinterpret_cast<T*>(smem + L::oV);
  T* sZ = reinterpret_cast<T*>(smem + L::oZ);
  float* sDec = reinterpret_cast<float*>(smem + L::oDec);

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int seg = blockIdx.x, unit = blockIdx.y;
  const int nchunks = (T_len + kC - 1) / kC;
  const int c_begin = seg * S;
  const int c_end = min(c_begin + S, nchunks);
  const T* kb = kk + (size_t)unit * T_len * DK;
  const T* vb = vv + (size_t)unit * T_len * DV;
  const T* gb = gg + (size_t)unit * T_len * M;

  f32x4 st[TPW];
#pragma unroll
  for (int s = 0; s < TPW; s++) st[s] = f32x4{0.f, 0.f, 0.f, 0.f};
  float segdec[SPT];
#pragma unroll
  for (int s = 0; s < SPT; s++) segdec[s] = 1.f;

  TileIO<T, DK> pk;
  TileIO<T, DV> pv;
  RowVec<T, SPT> pg;
  {
    int t0 = c_begin * kC, rv = min(kC, T_len - t0);
    pk.load(kb + (size_t)t0 * DK, rv, tid);
    pv.load(vb + (size_t)t0 * DV, rv, tid);
    pg.load(gb + (size_t)(t0 + lane) * M + wv * SPT, lane < rv);
  }
  for (int ch = c_begin; ch < c_end; ch++) {
    const int t0 = ch * kC, rv = min(kC, T_len - t0);
    pk.store_lds(sK, L::LDK, tid);
    pv.store_lds(sV, L::LDV, tid);
    Gates<SPT> gt;
    gt.compute(pg.v, lane < rv, inv_tau, lane);
#pragma unroll
    for (int s = 0; s < SPT; s++) {
      sZ[lane * L::LDM + wv * SPT + s] = Elem<T>::from_f(gt.w[s] * gt.Sx[s]);
      float d = __shfl(gt.E[s], 63, 64);
      if (lane == 0) sDec[wv * SPT + s] = d;
      segdec[s] *= d;
    }
    if (ch + 1 < c_end) {
      int t1 = t0 + kC, rv1 = min(kC, T_len - t1);
      pk.load(kb + (size_t)t1 * DK, rv1, tid);
      pv.load(vb + (size_t)t1 * DV, rv1, tid);
      pg.load(gb + (size_t)(t1 + lane) * M + wv * SPT, lane < rv1);
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < TPW; s++) {
      const int t = wv + kNW * s;
      if (t < NTS) {
        const int cb = t / NCT, nt = t % NCT;
#pragma unroll
        for (int i = 0; i < 4; i++) st[s][i] *= sDec[16 * cb + 4 * (lane >> 4) + i];
#pragma unroll
        for (int r0 = 0; r0 < kC; r0 += O::KS) {
          typename O::Frag fa = O::ld_t(sZ, L::LDM, 16 * cb, r0, lane);
          typename O::Frag fb = (nt < DK / 16) ? O::ld_t(sK, L::LDK, 16 * nt, r0, lane)
                                               : O::ld_t(sV, L::LDV, 16 * (nt - DK / 16), r0, lane);
          st[s] = O::mma(fa, fb, st[s]);
        }
      }
    }
    __syncthreads();
  }
  // write the map: state [M][DK+DV] then decay [M]
  float* out = ws_state + ((size_t)unit * P + seg) * M * (DK + DV);
#pragma unroll
  for (int s = 0; s < TPW; s++) {
    const int t = wv + kNW * s;
    if (t < NTS) {
      const int cb = t / NCT, nt = t % NCT;
#pragma unroll
      for (int i = 0; i < 4; i++)
        out[(16 * cb + 4 * (lane >> 4) + i) * (DK + DV) + 16 * nt + (lane & 15)] = st[s][i];
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int s = 0; s < SPT; s++) ws_dec[((size_t)unit * P + seg) * M + wv * SPT + s] = segdec[s];
  }
}

// ------------------------------------------------------- phase B: scan
// One thread per (unit, state element), serial over segments.  Slot p of the
// workspace holds segment p's map on entry (p < P-1) and its start state on
// exit; the last segment's workgroup in phase C produces the final state.
template <int DK, int DV, int M>
__global__ void __launch_bounds__(256)
gsa_seg_scan(float* __restrict__ ws_state, const float* __restrict__ ws_dec,
             const float* __restrict__ k0, const float* __restrict__ v0, int units, int P) {
  constexpr int NE = M * (DK + DV);
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long long)units * NE) return;
  const int unit = (int)(gid / NE), e = (int)(gid % NE);
  const int c = e / (DK + DV), col = e % (DK + DV);
  float W = 0.f;
  if (col < DK) {
    if (k0) W = k0[((size_t)unit * M + c) * DK + col];
  } else {
    if (v0) W = v0[((size_t)unit * M + c) * DV + col - DK];
  }
  float* st = ws_state + (size_t)unit * P * NE + e;
  const float* dc = ws_dec + (size_t)unit * P * M + c;
  for (int p = 0; p + 1 < P; p++) {
    const float x = st[(size_t)p * NE];
    st[(size_t)p * NE] = W;
    W = dc[(size_t)p * M] * W + x;
  }
  st[(size_t)(P - 1) * NE] = W;
}

// ---------------------------------------------------- phase C: outputs
template <typename T, int DK, int DV, int M, int ACT>
__global__ void __launch_bounds__(kNT, 1)
gsa_seg_out(const T* __restrict__ qq, const T* __restrict__ kk, const T* __restrict__ vv,
            const T* __restrict__ gg, const float* __restrict__ k0, const float* __restrict__ v0,
            const float* __restrict__ ws_state, T* __restrict__ oo, float* __restrict__ kf,
            float* __restrict__ vf, int T_len, int S, int P, float inv_tau) {
  using L = GsaLds<T, DK, DV, M>;
  using O = Op<T>;
  constexpr int SPT = M / kNW;
  constexpr int MT = M / 16;                 // slot tiles
  constexpr int NCT = (DK + DV) / 16;        // state column tiles
  constexpr int NTS = MT * NCT;              // state tiles
  constexpr int TPW = (NTS + kNW - 1) / kNW;
  constexpr int NT1 = (kC / 16) * MT;        // o' tiles
  constexpr int T1W = (NT1 + kNW - 1) / kNW;
  constexpr int NTO = (kC / 16) * (DV / 16);  // o tiles
  constexpr int TOW = (NTO + kNW - 1) / kNW;
  constexpr int NTA = (kC / 16) * (kC / 16 + 1) / 2;  // causal score tiles
  constexpr int TAW = (NTA + kNW - 1) / kNW;
  static_assert(SPT >= 1 && M % 16 == 0 && M >= O::KS && DK % 16 == 0 && DV % 16 == 0, "shape");

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  T* sQ = reinterpret_cast<T*>(smem + L::oQ);
  T* sK = reinterpret_cast<T*>(smem + L::oK);
  T* sV = reinterpret_cast<T*>(smem + L::oV);
  T* sW = reinterpret_cast<T*>(smem + L::oW);
  float* sE = reinterpret_cast<float*>(smem + L::oE);
  T* sX = reinterpret_cast<T*>(smem + L::oX);
  T* sZ = reinterpret_cast<T*>(smem + L::oZ);
  T* sSE = reinterpret_cast<T*>(smem + L::oSE);
  float* sAl = reinterpret_cast<float*>(smem + L::oAl);
  float* sWr = reinterpret_cast<float*>(smem + L::oWr);
  T* sA = reinterpret_cast<T*>(smem + L::oA);
  float* sRed = reinterpret_cast<float*>(smem + L::oRed);
  float* sRed2 = sRed + kC * MT;
  float* sDec = reinterpret_cast<float*>(smem + L::oDec);
  float* sZp = reinterpret_cast<float*>(smem + L::oZp);
  float* sOp = reinterpret_cast<float*>(smem + L::oOp);
  float* sS = reinterpret_cast<float*>(smem + L::oS);

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int seg = blockIdx.x, unit = blockIdx.y;
  const int nchunks = (T_len + kC - 1) / kC;
  const int c_begin = seg * S;
  const int c_end = min(c_begin + S, nchunks);
  const size_t ub = (size_t)unit * T_len;
  const T* qb = qq + ub * DK;
  const T* kb = kk + ub * DK;
  const T* vb = vv + ub * DV;
  const T* gb = gg + ub * M;
  T* ob = oo + ub * DV;

  // causal score buffer: zero once (only lower tiles are ever rewritten)
  for (int i = tid; i < kC * L::LDC; i += kNT) sA[i] = Elem<T>::from_f(0.f);

  // ---- start state into the MFMA accumulators
  f32x4 st[TPW];
#pragma unroll
  for (int s = 0; s < TPW; s++) {
    const int t = wv + kNW * s;
    st[s] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (t < NTS) {
      const int cb = t / NCT, nt = t % NCT;
      const int col = 16 * nt + (lane & 15);
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int c = 16 * cb + 4 * (lane >> 4) + i;
        float x = 0.f;
        if (P > 1) {
          x = ws_state[((size_t)unit * P + seg) * M * (DK + DV) + (size_t)c * (DK + DV) + col];
        } else if (col < DK) {
          if (k0) x = k0[((size_t)unit * M + c) * DK + col];
        } else {
          if (v0) x = v0[((size_t)unit * M + c) * DV + col - DK];
        }
        st[s][i] = x;
      }
    }
  }
  // op-dtype copy of the state for the read contractions
  auto write_state_copy = [&]() {
#pragma unroll
    for (int s = 0; s < TPW; s++) {
      const int t = wv + kNW * s;
      if (t < NTS) {
        const int cb = t / NCT, nt = t % NCT;
#pragma unroll
        for (int i = 0; i < 4; i++)
          sW[(16 * cb + 4 * (lane >> 4) + i) * L::LDW + 16 * nt + (lane & 15)] =
              Elem<T>::from_f(st[s][i]);
      }
    }
  };
  write_state_copy();

  TileIO<T, DK> pq, pk;
  TileIO<T, DV> pv;
  RowVec<T, SPT> pg;
  {
    const int t0 = c_begin * kC, rv = min(kC, T_len - t0);
    pq.load(qb + (size_t)t0 * DK, rv, tid);
    pk.load(kb + (size_t)t0 * DK, rv, tid);
    pv.load(vb + (size_t)t0 * DV, rv, tid);
    pg.load(gb + (size_t)(t0 + lane) * M + wv * SPT, lane < rv);
  }

  for (int ch = c_begin; ch < c_end; ch++) {
    const int t0 = ch * kC, rv = min(kC, T_len - t0);
    pq.store_lds(sQ, L::LDK, tid);
    pk.store_lds(sK, L::LDK, tid);
    pv.store_lds(sV, L::LDV, tid);
    Gates<SPT> gt;
    gt.compute(pg.v, lane < rv, inv_tau, lane);
    bool small = false;
#pragma unroll
    for (int s = 0; s < SPT; s++) small |= (gt.E[s] < kFastMinDecay);
    const bool slow = __syncthreads_or((lane == 63) && small) != 0;
    if (!slow) {
#pragma unroll
      for (int s = 0; s < SPT; s++) {
        const int c = wv * SPT + s;
        const float e = gt.E[s];
        sE[lane * L::LDE + c] = e;
        sX[lane * L::LDM + c] = Elem<T>::from_f(gt.w[s] / e);
        sZ[lane * L::LDM + c] = Elem<T>::from_f(gt.w[s] * gt.Sx[s]);
        const float d = __shfl(e, 63, 64);
        if (lane == 0) sDec[c] = d;
      }
    } else {
#pragma unroll
      for (int s = 0; s < SPT; s++) {
        const int c = wv * SPT + s;
        sAl[lane * M + c] = gt.a[s];
        sWr[lane * M + c] = gt.w[s];
      }
    }
    if (ch + 1 < c_end) {  // prefetch the next chunk into registers
      const int t1 = t0 + kC, rv1 = min(kC, T_len - t1);
      pq.load(qb + (size_t)t1 * DK, rv1, tid);
      pk.load(kb + (size_t)t1 * DK, rv1, tid);
      pv.load(vb + (size_t)t1 * DV, rv1, tid);
      pg.load(gb + (size_t)(t1 + lane) * M + wv * SPT, lane < rv1);
    }
    __syncthreads();

    if (!slow) {
      // ---- pass 1: causal scores A = mask(Q K^T)
#pragma unroll
      for (int s = 0; s < TAW; s++) {
        const int t = wv + kNW * s;
        if (t < NTA) {
          int J = 0, R = t;
          while (R > J) { R -= J + 1; J++; }
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int k0_ = 0; k0_ < DK; k0_ += O::KS)
            acc = O::mma(O::ld_k(sQ, L::LDK, 16 * J, k0_, lane), O::ld_k(sK, L::LDK, 16 * R, k0_, lane), acc);
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const int row = 16 * J + 4 * (lane >> 4) + i, col = 16 * R + (lane & 15);
            sA[row * L::LDC + col] = Elem<T>::from_f(col <= row ? acc[i] : 0.f);
          }
        }
      }
      // ---- pass 1: inter-chunk read Q Wk^T
      f32x4 a1[T1W];
#pragma unroll
      for (int s = 0; s < T1W; s++) {
        const int t = wv + kNW * s;
        a1[s] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (t < NT1) {
          const int J = t / MT, ct = t % MT;
#pragma unroll
          for (int k0_ = 0; k0_ < DK; k0_ += O::KS)
            a1[s] = O::mma(O::ld_k(sQ, L::LDK, 16 * J, k0_, lane), O::ld_k(sW, L::LDW, 16 * ct, k0_, lane), a1[s]);
        }
      }
      __syncthreads();
      // ---- pass 1: intra term A (I / E) and scaling by E; row maxima
#pragma unroll
      for (int s = 0; s < T1W; s++) {
        const int t = wv + kNW * s;
        if (t < NT1) {
          const int J = t / MT, ct = t % MT;
          const int rend = 16 * J + 16;
#pragma unroll
          for (int r0 = 0; r0 < kC; r0 += O::KS)
            if (r0 < rend)
              a1[s] = O::mma(O::ld_k(sA, L::LDC, 16 * J, r0, lane), O::ld_t(sX, L::LDM, 16 * ct, r0, lane), a1[s]);
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const int row = 16 * J + 4 * (lane >> 4) + i, col = 16 * ct + (lane & 15);
            a1[s][i] *= sE[row * L::LDE + col];
            if constexpr (ACT == kActSoftmax) {
              const float mx = max16(a1[s][i]);
              if ((lane & 15) == 0) sRed[row * MT + ct] = mx;
            }
          }
        }
      }
      __syncthreads();
      // ---- slot softmax: exp and row sums (the element-wise ablation
      // functions need neither)
#pragma unroll
      for (int s = 0; s < T1W; s++) {
        const int t = wv + kNW * s;
        if (ACT == kActSoftmax && t < NT1) {
          const int J = t / MT, ct = t % MT;
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const int row = 16 * J + 4 * (lane >> 4) + i;
            float mx = sRed[row * MT];
#pragma unroll
            for (int c2 = 1; c2 < MT; c2++) mx = fmaxf(mx, sRed[row * MT + c2]);
            a1[s][i] = __expf(a1[s][i] - mx);
            const float sm = sum16(a1[s][i]);
            if ((lane & 15) == 0) sRed2[row * MT + ct] = sm;
          }
        }
      }
      __syncthreads();
#pragma unroll
      for (int s = 0; s < T1W; s++) {
        const int t = wv + kNW * s;
        if (t < NT1) {
          const int J = t / MT, ct = t % MT;
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const int row = 16 * J + 4 * (lane >> 4) + i, col = 16 * ct + (lane & 15);
            float sv;
            if constexpr (ACT == kActSoftmax) {
              float sm = 0.f;
#pragma unroll
              for (int c2 = 0; c2 < MT; c2++) sm += sRed2[row * MT + c2];
              sv = a1[s][i] / sm;
            } else {
              sv = slot_act<ACT>(a1[s][i]);
            }
            sSE[row * L::LDM + col] = Elem<T>::from_f(sv * sE[row * L::LDE + col]);
          }
        }
      }
      __syncthreads();
      // ---- pass 2: causal scores A2 = mask((s*E) (I/E)^T)
#pragma unroll
      for (int s = 0; s < TAW; s++) {
        const int t = wv + kNW * s;
        if (t < NTA) {
          int J = 0, R = t;
          while (R > J) { R -= J + 1; J++; }
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int c0 = 0; c0 < M; c0 += O::KS)
            acc = O::mma(O::ld_k(sSE, L::LDM, 16 * J, c0, lane), O::ld_k(sX, L::LDM, 16 * R, c0, lane), acc);
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const int row = 16 * J + 4 * (lane >> 4) + i, col = 16 * R + (lane & 15);
            sA[row * L::LDC + col] = Elem<T>::from_f(col <= row ? acc[i] : 0.f);
          }
        }
      }
      __syncthreads();
      // ---- pass 2: o = (s*E) Wv + A2 V
#pragma unroll
      for (int s = 0; s < TOW; s++) {
        const int t = wv + kNW * s;
        if (t < NTO) {
          const int J = t / (DV / 16), nt = t % (DV / 16);
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int c0 = 0; c0 < M; c0 += O::KS)
            acc = O::mma(O::ld_k(sSE, L::LDM, 16 * J, c0, lane), O::ld_t(sW + DK, L::LDW, 16 * nt, c0, lane), acc);
          const int rend = 16 * J + 16;
#pragma unroll
          for (int r0 = 0; r0 < kC; r0 += O::KS)
            if (r0 < rend)
              acc = O::mma(O::ld_k(sA, L::LDC, 16 * J, r0, lane), O::ld_t(sV, L::LDV, 16 * nt, r0, lane), acc);
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const int row = 16 * J + 4 * (lane >> 4) + i;
            if (row < rv) ob[(size_t)(t0 + row) * DV + 16 * nt + (lane & 15)] = Elem<T>::from_f(acc[i]);
          }
        }
      }
      // ---- state carry: W <- Diag(prod alpha) W + (I*S)^T [K|V]
#pragma unroll
      for (int s = 0; s < TPW; s++) {
        const int t = wv + kNW * s;
        if (t < NTS) {
          const int cb = t / NCT, nt = t % NCT;
#pragma unroll
          for (int i = 0; i < 4; i++) st[s][i] *= sDec[16 * cb + 4 * (lane >> 4) + i];
#pragma unroll
          for (int r0 = 0; r0 < kC; r0 += O::KS) {
            typename O::Frag fa = O::ld_t(sZ, L::LDM, 16 * cb, r0, lane);
            typename O::Frag fb = (nt < DK / 16) ? O::ld_t(sK, L::LDK, 16 * nt, r0, lane)
                                                 : O::ld_t(sV, L::LDV, 16 * (nt - DK / 16), r0, lane);
            st[s] = O::mma(fa, fb, st[s]);
          }
        }
      }
    } else {
      // ---- exact token recurrence on the register-resident state
      for (int j = 0; j < rv; j++) {
        const T* qj = sQ + j * L::LDK;
        const T* kj = sK + j * L::LDK;
        const T* vj = sV + j * L::LDV;
#pragma unroll
        for (int s = 0; s < TPW; s++) {
          const int t = wv + kNW * s;
          if (t < NTS) {
            const int cb = t / NCT, nt = t % NCT;
            const int col = 16 * nt + (lane & 15);
            const float x = (nt < DK / 16) ? Elem<T>::to_f(kj[col]) : Elem<T>::to_f(vj[col - DK]);
            float zpart[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
              const int c = 16 * cb + 4 * (lane >> 4) + i;
              st[s][i] = sAl[j * M + c] * st[s][i] + sWr[j * M + c] * x;
              zpart[i] = (nt < DK / 16) ? st[s][i] * Elem<T>::to_f(qj[col]) : 0.f;
            }
            if (nt < DK / 16) {
#pragma unroll
              for (int i = 0; i < 4; i++) {
                const float zs = sum16(zpart[i]);
                if ((lane & 15) == 0) sZp[nt * M + 16 * cb + 4 * (lane >> 4) + i] = zs;
              }
            }
          }
        }
        __syncthreads();
        if (wv == 0) {
          float z = -INFINITY;
          if (lane < M) {
            z = 0.f;
#pragma unroll
            for (int nt = 0; nt < DK / 16; nt++) z += sZp[nt * M + lane];
          }
          if constexpr (ACT == kActSoftmax) {
            float mx = z;
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
            const float e = (lane < M) ? __expf(z - mx) : 0.f;
            const float sm = sum64(e);
            if (lane < M) sS[lane] = e / sm;
          } else {
            if (lane < M) sS[lane] = slot_act<ACT>(z);
          }
        }
        __syncthreads();
#pragma unroll
        for (int s = 0; s < TPW; s++) {
          const int t = wv + kNW * s;
          if (t < NTS) {
            const int cb = t / NCT, nt = t % NCT;
            if (nt >= DK / 16) {
              float p = 0.f;
#pragma unroll
              for (int i = 0; i < 4; i++) p += st[s][i] * sS[16 * cb + 4 * (lane >> 4) + i];
              p += __shfl_xor(p, 16, 64);
              p += __shfl_xor(p, 32, 64);
              if (lane < 16) sOp[cb * DV + 16 * (nt - DK / 16) + lane] = p;
            }
          }
        }
        __syncthreads();
        for (int n = tid; n < DV; n += kNT) {
          float acc = 0.f;
#pragma unroll
          for (int cb = 0; cb < MT; cb++) acc += sOp[cb * DV + n];
          ob[(size_t)(t0 + j) * DV + n] = Elem<T>::from_f(acc);
        }
      }
    }
    __syncthreads();
    write_state_copy();
  }

  if (seg == P - 1) {  // the last segment's workgroup ends holding the final state
#pragma unroll
    for (int s = 0; s < TPW; s++) {
      const int t = wv + kNW * s;
      if (t < NTS) {
        const int cb = t / NCT, nt = t % NCT;
        const int col = 16 * nt + (lane & 15);
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int c = 16 * cb + 4 * (lane >> 4) + i;
          if (col < DK) {
            if (kf) kf[((size_t)unit * M + c) * DK + col] = st[s][i];
          } else {
            if (vf) vf[((size_t)unit * M + c) * DV + col - DK] = st[s][i];
          }
        }
      }
    }
  }
}

// ------------------------------------------------------------ launcher
template <typename T, int DK, int DV, int M, int ACT>
static int launch_gsa(const GsaLaunch& a) {
  using LO = GsaLds<T, DK, DV, M>;
  using LS = GsaStateLds<T, DK, DV, M>;
  const int units = a.B * a.H;
  const int nchunks = (a.T + kC - 1) / kC;
  const int S = a.chunks_per_seg;
  const int P = (nchunks + S - 1) / S;
  const float inv_tau = 1.0f / a.tau;
  hipStream_t st = (hipStream_t)a.stream;
  if (P > 1) {
    launch_timed(gsa_seg_state<T, DK, DV, M>, dim3(P - 1, units), dim3(kNT), LS::total, a.stream,
                 a.events, 0, 1, (const T*)a.k, (const T*)a.v, (const T*)a.g, a.ws_state, a.ws_dec,
                 a.T, S, P, inv_tau);
    const long long ne = (long long)units * M * (DK + DV);
    hipLaunchKernelGGL((gsa_seg_scan<DK, DV, M>), dim3((unsigned)((ne + 255) / 256)), dim3(256), 0, st,
                       a.ws_state, (const float*)a.ws_dec, a.k0, a.v0, units, P);
  } else {
    record_event(a.events, 0, a.stream);
    record_event(a.events, 1, a.stream);
  }
  launch_timed(gsa_seg_out<T, DK, DV, M, ACT>, dim3(P, units), dim3(kNT), LO::total, a.stream, a.events, 2,
               3, (const T*)a.q, (const T*)a.k, (const T*)a.v, (const T*)a.g, a.k0, a.v0,
               (const float*)a.ws_state, (T*)a.o, a.kf, a.vf, a.T, S, P, inv_tau);
  return 0;
}

template <typename T, int DK, int DV, int M, int ACT>
static void set_lds_limits() {
  (void)hipFuncSetAttribute((const void*)gsa_seg_out<T, DK, DV, M, ACT>,
                      hipFuncAttributeMaxDynamicSharedMemorySize, GsaLds<T, DK, DV, M>::total);
  (void)hipFuncSetAttribute((const void*)gsa_seg_state<T, DK, DV, M>,
                      hipFuncAttributeMaxDynamicSharedMemorySize, GsaStateLds<T, DK, DV, M>::total);
}

template <typename T, int DK, int DV, int M>
constexpr bool gsa_fits() {
  return GsaLds<T, DK, DV, M>::total <= kLdsBytes;
}

template <typename T, int DK, int DV, int M>
static int launch_gsa_act(const GsaLaunch& a) {
  switch (a.act) {
#define GSA_ACT_CASE(A)               \
  case A:                             \
    set_lds_limits<T, DK, DV, M, A>(); \
    return launch_gsa<T, DK, DV, M, A>(a);
    GSA_ACT_CASE(kActSoftmax)
    GSA_ACT_CASE(kActIdentity)
    GSA_ACT_CASE(kActSwish)
    GSA_ACT_CASE(kActRelu)
    GSA_ACT_CASE(kActRelu2)
#undef GSA_ACT_CASE
    default: return -1;
  }
}

#define GSA_CASE(TT, DTC, DKC, DVC, MC)                                                   \
  if (dt == DTC && dk == DKC && dv == DVC && m == MC) {                                 \
    if constexpr (gsa_fits<TT, DKC, DVC, MC>()) {                                        \
      if (query) return GsaLds<TT, DKC, DVC, MC>::total;                                 \
      return launch_gsa_act<TT, DKC, DVC, MC>(*a);                                       \
    }                                                                                    \
    return -1;                                                                           \
  }

// Returns: query -> LDS bytes (>0) or -1 if unsupported; launch -> 0 or -1.
// bf16 inputs take the kernels of gsa_fwd_bf16.hip; this file serves float32.
int gsa_dispatch(int dt, int dk, int dv, int m, const GsaLaunch* a, bool query) {
  if (dt == 1) return gsa_dispatch_bf16(dk, dv, m, a, query);
  GSA_CASE(float, 0, 64, 64, 64)
  GSA_CASE(float, 0, 64, 64, 32)
  GSA_CASE(float, 0, 64, 64, 16)
  GSA_CASE(float, 0, 128, 128, 32)
  GSA_CASE(float, 0, 128, 128, 16)
  return -1;
}

}  // namespace gsa
