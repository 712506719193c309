// Chunkwise gated linear attention (GLA) forward on gfx950.
//
// Method: "Gated Slot Attention for Efficient Linear-Time Sequence Modeling",
// Sec. 2.3 (GLA with beta = 1) and App. A.1 (chunkwise form):
//   S_t = Diag(alpha_t) S_{t-1} + k_t v_t^T,   o_t = S_t^T q_t,
//   alpha_t = sigmoid(g_t)^(1/tau) per key dimension, S in R^{dk x dv}.
// Within a chunk, with E_j = prod_{i<=j} alpha_i and S_r = prod_{i>r} alpha_i
// (per key dimension):
//   o_j = (q_j * E_j)^T S_0 + sum_{r<=j} [(q_j*E_j) . (k_r/E_r)] v_r
//   S   <- Diag(E_C) S_0 + (K * S)^T V
// Same launch structure as the GSA forward: segment state maps (A), a serial
// fp32 scan over segments (B), and per-segment output recomputation (C), with
// an exact token-recurrence path for chunks whose decay product drops below
// e^-40 in some key dimension.
#include "common.hpp"
#include "internal.hpp"
#include "launch.hpp"

namespace gsa {

constexpr int gC = 64;
constexpr int gNW = 8;
constexpr int gNT = gNW * 64;

template <typename T, int DK, int DV>
struct GlaLds {
  static constexpr int PAD = Pad<T>::v;
  static constexpr int LDK = DK + PAD, LDV = DV + PAD, LDC = gC + PAD, LDS_ = DK + PAD;
  static constexpr int TS = (int)sizeof(T);
  static constexpr int oV = 0;
  static constexpr int oS = oV + gC * LDV * TS;            // state copy [DV][DK]
  static constexpr int oU = oS + DV * LDS_ * TS;
  // fast: QE, KX, KZ ([C][LDK] T) and causal scores [C][LDC] T
  static constexpr int oQE = oU;
  static constexpr int oKX = oQE + gC * LDK * TS;
  static constexpr int oKZ = oKX + gC * LDK * TS;
  static constexpr int oA = oKZ + gC * LDK * TS;
  static constexpr int szFast = 3 * gC * LDK * TS + gC * LDC * TS;
  // slow: alpha fp32 [C][DK], raw q, k [C][LDK] T
  static constexpr int oAl = oU;
  static constexpr int oQr = oAl + gC * DK * 4;
  static constexpr int oKr = oQr + gC * LDK * TS;
  static constexpr int szSlow = gC * DK * 4 + 2 * gC * LDK * TS;
  static constexpr int szU = szFast > szSlow ? szFast : szSlow;
  static constexpr int oDec = oU + szU;                     // [DK] fp32
  static constexpr int oOp = oDec + DK * 4;                 // [DK/16][DV] fp32
  static constexpr int total = oOp + (DK / 16) * DV * 4;
  static_assert(oS % 16 == 0 && oU % 16 == 0 && oKX % 16 == 0 && oKZ % 16 == 0 && oA % 16 == 0 &&
                    oQr % 16 == 0 && oKr % 16 == 0 && oDec % 16 == 0,
                "alignment");
};

template <typename T, int DK, int DV>
struct GlaStateLds {
  static constexpr int PAD = Pad<T>::v;
  static constexpr int LDK = DK + PAD, LDV = DV + PAD;
  static constexpr int TS = (int)sizeof(T);
  static constexpr int oV = 0;
  static constexpr int oKZ = oV + gC * LDV * TS;
  static constexpr int oDec = oKZ + gC * LDK * TS;
  static constexpr int total = oDec + DK * 4;
};

template <typename T, int D>
struct GTile {  // [C][D] tile moved as 16-byte vectors by 512 threads
  static constexpr int VPR = D * (int)sizeof(T) / 16;
  static constexpr int NV = gC * VPR / gNT;
  static constexpr int EPV = 16 / (int)sizeof(T);
  static_assert(NV >= 1 && (gC * VPR) % gNT == 0, "tile/thread mismatch");
  uint4 r[NV];
  __device__ __forceinline__ void load(const T* __restrict__ base, int rows_valid, int tid) {
#pragma unroll
    for (int i = 0; i < NV; i++) {
      int idx = tid + gNT * i, row = idx / VPR, cv = idx % VPR;
      r[i] = (row < rows_valid) ? *reinterpret_cast<const uint4*>(base + (size_t)row * D + cv * EPV)
                                : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store_lds(T* dst, int ld, int tid) const {
#pragma unroll
    for (int i = 0; i < NV; i++) {
      int idx = tid + gNT * i, row = idx / VPR, cv = idx % VPR;
      *reinterpret_cast<uint4*>(dst + row * ld + cv * EPV) = r[i];
    }
  }
};

// DPT consecutive elements of one row as raw 16-byte vectors (N*sizeof(T) % 16 == 0)
template <typename T, int N>
struct GRow {
  static constexpr int NV = N * (int)sizeof(T) / 16;
  static_assert(NV >= 1 && (N * (int)sizeof(T)) % 16 == 0, "row vector");
  uint4 r[NV];
  __device__ __forceinline__ void load(const T* __restrict__ p, bool valid) {
#pragma unroll
    for (int i = 0; i < NV; i++)
      r[i] = valid ? *reinterpret_cast<const uint4*>(p + i * (16 / (int)sizeof(T))) : make_uint4(0, 0, 0, 0);
  }
  __device__ __forceinline__ float at(int s) const { return Elem<T>::to_f(reinterpret_cast<const T*>(r)[s]); }
};

template <int DPT, int GM>
struct GlaGates {
  float a[DPT], E[DPT], Sx[DPT];
  __device__ __forceinline__ void compute(const float* g, bool valid, float inv_tau, int lane) {
#pragma unroll
    for (int s = 0; s < DPT; s++) {
      // a logit (alpha = sigmoid(g)^(1/tau)) or a log-decay given directly
      const float al = GM == kGateLogit ? gate_alpha(g[s], inv_tau) : __expf(fminf(g[s], 0.f));
      a[s] = valid ? al : 1.f;
      E[s] = a[s];
      Sx[s] = a[s];
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
#pragma unroll
      for (int s = 0; s < DPT; s++) {
        float up = __shfl_up(E[s], off, 64);
        float dn = __shfl_down(Sx[s], off, 64);
        if (lane >= off) E[s] *= up;
        if (lane + off < 64) Sx[s] *= dn;
      }
    }
#pragma unroll
    for (int s = 0; s < DPT; s++) {
      float nx = __shfl_down(Sx[s], 1, 64);
      Sx[s] = (lane == 63) ? 1.f : nx;
    }
  }
};

// ------------------------------------------------------ phase A: state map
template <typename T, int DK, int DV, int GM>
__global__ void __launch_bounds__(gNT, 1)
gla_seg_state(const T* __restrict__ kk, const T* __restrict__ vv, const T* __restrict__ gg,
              float* __restrict__ ws_state, float* __restrict__ ws_dec, int T_len, int S, int P,
              float inv_tau) {
  using L = GlaStateLds<T, DK, DV>;
  using O = Op<T>;
  constexpr int DPT = DK / gNW;
  constexpr int NCT = DV / 16;
  constexpr int NTS = (DK / 16) * NCT;
  constexpr int TPW = (NTS + gNW - 1) / gNW;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  T* sV = reinterpret_cast<T*>(smem + L::oV);
  T* sKZ = reinterpret_cast<T*>(smem + L::oKZ);
  float* sDec = reinterpret_cast<float*>(smem + L::oDec);

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int seg = blockIdx.x, unit = blockIdx.y;
  const int nchunks = (T_len + gC - 1) / gC;
  const int c_begin = seg * S, c_end = min(c_begin + S, nchunks);
  const T* kb = kk + (size_t)unit * T_len * DK;
  const T* vb = vv + (size_t)unit * T_len * DV;
  const T* gb = gg + (size_t)unit * T_len * DK;

  f32x4 st[TPW];
#pragma unroll
  for (int s = 0; s < TPW; s++) st[s] = f32x4{0.f, 0.f, 0.f, 0.f};
  float segdec[DPT];
#pragma unroll
  for (int s = 0; s < DPT; s++) segdec[s] = 1.f;

  GTile<T, DV> pv;
  GRow<T, DPT> pk, pg;
  {
    const int t0 = c_begin * gC, rv = min(gC, T_len - t0);
    pv.load(vb + (size_t)t0 * DV, rv, tid);
    pk.load(kb + (size_t)(t0 + lane) * DK + wv * DPT, lane < rv);
    pg.load(gb + (size_t)(t0 + lane) * DK + wv * DPT, lane < rv);
  }
  for (int ch = c_begin; ch < c_end; ch++) {
    const int t0 = ch * gC, rv = min(gC, T_len - t0);
    pv.store_lds(sV, L::LDV, tid);
    float gv[DPT];
#pragma unroll
    for (int s = 0; s < DPT; s++) gv[s] = pg.at(s);
    GlaGates<DPT, GM> gt;
    gt.compute(gv, lane < rv, inv_tau, lane);
#pragma unroll
    for (int s = 0; s < DPT; s++) {
      const int c = wv * DPT + s;
      sKZ[lane * L::LDK + c] = Elem<T>::from_f(pk.at(s) * gt.Sx[s]);
      const float d = __shfl(gt.E[s], 63, 64);
      if (lane == 0) sDec[c] = d;
      segdec[s] *= d;
    }
    if (ch + 1 < c_end) {
      const int t1 = t0 + gC, rv1 = min(gC, T_len - t1);
      pv.load(vb + (size_t)t1 * DV, rv1, tid);
      pk.load(kb + (size_t)(t1 + lane) * DK + wv * DPT, lane < rv1);
      pg.load(gb + (size_t)(t1 + lane) * DK + wv * DPT, lane < rv1);
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < TPW; s++) {
      const int t = wv + gNW * s;
      if (t < NTS) {
        const int cb = t / NCT, nt = t % NCT;
#pragma unroll
        for (int i = 0; i < 4; i++) st[s][i] *= sDec[16 * cb + 4 * (lane >> 4) + i];
#pragma unroll
        for (int r0 = 0; r0 < gC; r0 += O::KS)
          st[s] = O::mma(O::ld_t(sKZ, L::LDK, 16 * cb, r0, lane), O::ld_t(sV, L::LDV, 16 * nt, r0, lane), st[s]);
      }
    }
    __syncthreads();
  }
  float* out = ws_state + ((size_t)unit * P + seg) * DK * DV;
#pragma unroll
  for (int s = 0; s < TPW; s++) {
    const int t = wv + gNW * s;
    if (t < NTS) {
      const int cb = t / NCT, nt = t % NCT;
#pragma unroll
      for (int i = 0; i < 4; i++)
        out[(16 * cb + 4 * (lane >> 4) + i) * DV + 16 * nt + (lane & 15)] = st[s][i];
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int s = 0; s < DPT; s++) ws_dec[((size_t)unit * P + seg) * DK + wv * DPT + s] = segdec[s];
  }
}

// ------------------------------------------------------- phase B: scan
// Slot p holds segment p's map on entry (p < P-1) and its start state on exit.
template <int DK, int DV>
__global__ void __launch_bounds__(256)
gla_seg_scan(float* __restrict__ ws_state, const float* __restrict__ ws_dec,
             const float* __restrict__ s0, int units, int P) {
  constexpr int NE = DK * DV;
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long long)units * NE) return;
  const int unit = (int)(gid / NE), e = (int)(gid % NE);
  const int c = e / DV;
  float W = s0 ? s0[(size_t)unit * NE + e] : 0.f;
  float* st = ws_state + (size_t)unit * P * NE + e;
  const float* dc = ws_dec + (size_t)unit * P * DK + c;
  for (int p = 0; p + 1 < P; p++) {
    const float x = st[(size_t)p * NE];
    st[(size_t)p * NE] = W;
    W = dc[(size_t)p * DK] * W + x;
  }
  st[(size_t)(P - 1) * NE] = W;
}

// ---------------------------------------------------- phase C: outputs
template <typename T, int DK, int DV, int GM>
__global__ void __launch_bounds__(gNT, 1)
gla_seg_out(const T* __restrict__ qq, const T* __restrict__ kk, const T* __restrict__ vv,
            const T* __restrict__ gg, const float* __restrict__ s0, const float* __restrict__ ws_state,
            T* __restrict__ oo, float* __restrict__ sf, int T_len, int S, int P, float inv_tau) {
  using L = GlaLds<T, DK, DV>;
  using O = Op<T>;
  constexpr int DPT = DK / gNW;
  constexpr int NCT = DV / 16;
  constexpr int NTS = (DK / 16) * NCT;
  constexpr int TPW = (NTS + gNW - 1) / gNW;
  constexpr int NTO = (gC / 16) * NCT;
  constexpr int TOW = (NTO + gNW - 1) / gNW;
  constexpr int NTA = (gC / 16) * (gC / 16 + 1) / 2;
  constexpr int TAW = (NTA + gNW - 1) / gNW;

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  T* sV = reinterpret_cast<T*>(smem + L::oV);
  T* sS = reinterpret_cast<T*>(smem + L::oS);
  T* sQE = reinterpret_cast<T*>(smem + L::oQE);
  T* sKX = reinterpret_cast<T*>(smem + L::oKX);
  T* sKZ = reinterpret_cast<T*>(smem + L::oKZ);
  T* sA = reinterpret_cast<T*>(smem + L::oA);
  float* sAl = reinterpret_cast<float*>(smem + L::oAl);
  T* sQr = reinterpret_cast<T*>(smem + L::oQr);
  T* sKr = reinterpret_cast<T*>(smem + L::oKr);
  float* sDec = reinterpret_cast<float*>(smem + L::oDec);
  float* sOp = reinterpret_cast<float*>(smem + L::oOp);

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int seg = blockIdx.x, unit = blockIdx.y;
  const int nchunks = (T_len + gC - 1) / gC;
  const int c_begin = seg * S, c_end = min(c_begin + S, nchunks);
  const size_t ub = (size_t)unit * T_len;
  const T* qb = qq + ub * DK;
  const T* kb = kk + ub * DK;
  const T* vb = vv + ub * DV;
  const T* gb = gg + ub * DK;
  T* ob = oo + ub * DV;

  f32x4 st[TPW];
#pragma unroll
  for (int s = 0; s < TPW; s++) {
    const int t = wv + gNW * s;
    st[s] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (t < NTS) {
      const int cb = t / NCT, nt = t % NCT;
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const size_t e = (size_t)(16 * cb + 4 * (lane >> 4) + i) * DV + 16 * nt + (lane & 15);
        float x = 0.f;
        if (P > 1) x = ws_state[((size_t)unit * P + seg) * DK * DV + e];
        else if (s0) x = s0[(size_t)unit * DK * DV + e];
        st[s][i] = x;
      }
    }
  }
  auto write_state_copy = [&]() {  // sS[n][c] = S[c][n]
#pragma unroll
    for (int s = 0; s < TPW; s++) {
      const int t = wv + gNW * s;
      if (t < NTS) {
        const int cb = t / NCT, nt = t % NCT;
#pragma unroll
        for (int i = 0; i < 4; i++)
          sS[(16 * nt + (lane & 15)) * L::LDS_ + 16 * cb + 4 * (lane >> 4) + i] = Elem<T>::from_f(st[s][i]);
      }
    }
  };
  bool zeroed_A = false;
  write_state_copy();

  GTile<T, DV> pv;
  GRow<T, DPT> pq, pk, pg;
  {
    const int t0 = c_begin * gC, rv = min(gC, T_len - t0);
    pv.load(vb + (size_t)t0 * DV, rv, tid);
    const size_t ro = (size_t)(t0 + lane) * DK + wv * DPT;
    pq.load(qb + ro, lane < rv);
    pk.load(kb + ro, lane < rv);
    pg.load(gb + ro, lane < rv);
  }
  for (int ch = c_begin; ch < c_end; ch++) {
    const int t0 = ch * gC, rv = min(gC, T_len - t0);
    pv.store_lds(sV, L::LDV, tid);
    float gv[DPT];
#pragma unroll
    for (int s = 0; s < DPT; s++) gv[s] = pg.at(s);
    GlaGates<DPT, GM> gt;
    gt.compute(gv, lane < rv, inv_tau, lane);
    bool small = false;
#pragma unroll
    for (int s = 0; s < DPT; s++) small |= (gt.E[s] < kFastMinDecay);
    const bool slow = __syncthreads_or((lane == 63) && small) != 0;
    if (!slow) {
      if (!zeroed_A) {  // the score buffer aliases slow-path storage: re-zero after slow use
        for (int i = tid; i < gC * L::LDC; i += gNT) sA[i] = Elem<T>::from_f(0.f);
        zeroed_A = true;
      }
#pragma unroll
      for (int s = 0; s < DPT; s++) {
        const int c = wv * DPT + s;
        const float e = gt.E[s];
        sQE[lane * L::LDK + c] = Elem<T>::from_f(pq.at(s) * e);
        sKX[lane * L::LDK + c] = Elem<T>::from_f(pk.at(s) / e);
        sKZ[lane * L::LDK + c] = Elem<T>::from_f(pk.at(s) * gt.Sx[s]);
        const float d = __shfl(e, 63, 64);
        if (lane == 0) sDec[c] = d;
      }
    } else {
      zeroed_A = false;
#pragma unroll
      for (int s = 0; s < DPT; s++) {
        const int c = wv * DPT + s;
        sAl[lane * DK + c] = gt.a[s];
        sQr[lane * L::LDK + c] = Elem<T>::from_f(pq.at(s));
        sKr[lane * L::LDK + c] = Elem<T>::from_f(pk.at(s));
      }
    }
    if (ch + 1 < c_end) {
      const int t1 = t0 + gC, rv1 = min(gC, T_len - t1);
      pv.load(vb + (size_t)t1 * DV, rv1, tid);
      const size_t ro = (size_t)(t1 + lane) * DK + wv * DPT;
      pq.load(qb + ro, lane < rv1);
      pk.load(kb + ro, lane < rv1);
      pg.load(gb + ro, lane < rv1);
    }
    __syncthreads();
    if (!slow) {
      // causal scores A = mask((Q*E)(K/E)^T)
#pragma unroll
      for (int s = 0; s < TAW; s++) {
        const int t = wv + gNW * s;
        if (t < NTA) {
          int J = 0, R = t;
          while (R > J) { R -= J + 1; J++; }
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int c0 = 0; c0 < DK; c0 += O::KS)
            acc = O::mma(O::ld_k(sQE, L::LDK, 16 * J, c0, lane), O::ld_k(sKX, L::LDK, 16 * R, c0, lane), acc);
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const int row = 16 * J + 4 * (lane >> 4) + i, col = 16 * R + (lane & 15);
            sA[row * L::LDC + col] = Elem<T>::from_f(col <= row ? acc[i] : 0.f);
          }
        }
      }
      __syncthreads();
      // o = (Q*E) S + A V
#pragma unroll
      for (int s = 0; s < TOW; s++) {
        const int t = wv + gNW * s;
        if (t < NTO) {
          const int J = t / NCT, nt = t % NCT;
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int c0 = 0; c0 < DK; c0 += O::KS)
            acc = O::mma(O::ld_k(sQE, L::LDK, 16 * J, c0, lane), O::ld_k(sS, L::LDS_, 16 * nt, c0, lane), acc);
          const int rend = 16 * J + 16;
#pragma unroll
          for (int r0 = 0; r0 < gC; r0 += O::KS)
            if (r0 < rend)
              acc = O::mma(O::ld_k(sA, L::LDC, 16 * J, r0, lane), O::ld_t(sV, L::LDV, 16 * nt, r0, lane), acc);
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const int row = 16 * J + 4 * (lane >> 4) + i;
            if (row < rv) ob[(size_t)(t0 + row) * DV + 16 * nt + (lane & 15)] = Elem<T>::from_f(acc[i]);
          }
        }
      }
      // S <- Diag(E_C) S + (K*S_excl)^T V
#pragma unroll
      for (int s = 0; s < TPW; s++) {
        const int t = wv + gNW * s;
        if (t < NTS) {
          const int cb = t / NCT, nt = t % NCT;
#pragma unroll
          for (int i = 0; i < 4; i++) st[s][i] *= sDec[16 * cb + 4 * (lane >> 4) + i];
#pragma unroll
          for (int r0 = 0; r0 < gC; r0 += O::KS)
            st[s] = O::mma(O::ld_t(sKZ, L::LDK, 16 * cb, r0, lane), O::ld_t(sV, L::LDV, 16 * nt, r0, lane), st[s]);
        }
      }
    } else {
      for (int j = 0; j < rv; j++) {
#pragma unroll
        for (int s = 0; s < TPW; s++) {
          const int t = wv + gNW * s;
          if (t < NTS) {
            const int cb = t / NCT, nt = t % NCT;
            const float vjn = Elem<T>::to_f(sV[j * L::LDV + 16 * nt + (lane & 15)]);
            float p = 0.f;
#pragma unroll
            for (int i = 0; i < 4; i++) {
              const int c = 16 * cb + 4 * (lane >> 4) + i;
              st[s][i] = sAl[j * DK + c] * st[s][i] + Elem<T>::to_f(sKr[j * L::LDK + c]) * vjn;
              p += st[s][i] * Elem<T>::to_f(sQr[j * L::LDK + c]);
            }
            p += __shfl_xor(p, 16, 64);
            p += __shfl_xor(p, 32, 64);
            if (lane < 16) sOp[cb * DV + 16 * nt + lane] = p;
          }
        }
        __syncthreads();
        for (int n = tid; n < DV; n += gNT) {
          float acc = 0.f;
#pragma unroll
          for (int cb = 0; cb < DK / 16; cb++) acc += sOp[cb * DV + n];
          ob[(size_t)(t0 + j) * DV + n] = Elem<T>::from_f(acc);
        }
        __syncthreads();
      }
    }
    __syncthreads();
    write_state_copy();
  }
  if (seg == P - 1 && sf) {
#pragma unroll
    for (int s = 0; s < TPW; s++) {
      const int t = wv + gNW * s;
      if (t < NTS) {
        const int cb = t / NCT, nt = t % NCT;
#pragma unroll
        for (int i = 0; i < 4; i++)
          sf[(size_t)unit * DK * DV + (size_t)(16 * cb + 4 * (lane >> 4) + i) * DV + 16 * nt + (lane & 15)] = st[s][i];
      }
    }
  }
}

template <typename T, int DK, int DV, int GM>
static int launch_gla(const GlaLaunch& a) {
  using LO = GlaLds<T, DK, DV>;
  using LS = GlaStateLds<T, DK, DV>;
  const int units = a.B * a.H;
  const int nchunks = (a.T + gC - 1) / gC;
  const int S = a.chunks_per_seg;
  const int P = (nchunks + S - 1) / S;
  const float inv_tau = 1.0f / a.tau;
  hipStream_t st = (hipStream_t)a.stream;
  if (P > 1) {
    launch_timed(gla_seg_state<T, DK, DV, GM>, dim3(P - 1, units), dim3(gNT), LS::total, a.stream, a.events,
                 0, 1, (const T*)a.k, (const T*)a.v, (const T*)a.g, a.ws_state, a.ws_dec, a.T, S, P,
                 inv_tau);
    const long long ne = (long long)units * DK * DV;
    hipLaunchKernelGGL((gla_seg_scan<DK, DV>), dim3((unsigned)((ne + 255) / 256)), dim3(256), 0, st,
                       a.ws_state, (const float*)a.ws_dec, a.s0, units, P);
  } else {
    record_event(a.events, 0, a.stream);
    record_event(a.events, 1, a.stream);
  }
  launch_timed(gla_seg_out<T, DK, DV, GM>, dim3(P, units), dim3(gNT), LO::total, a.stream, a.events, 2, 3,
               (const T*)a.q, (const T*)a.k, (const T*)a.v, (const T*)a.g, a.s0,
               (const float*)a.ws_state, (T*)a.o, a.sf, a.T, S, P, inv_tau);
  return 0;
}

template <typename T, int DK, int DV>
constexpr bool gla_fits() { return GlaLds<T, DK, DV>::total <= kLdsBytes; }

template <typename T, int DK, int DV, int GM>
static int launch_gla_mode(const GlaLaunch& a) {
  (void)hipFuncSetAttribute((const void*)gla_seg_out<T, DK, DV, GM>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, GlaLds<T, DK, DV>::total);
  (void)hipFuncSetAttribute((const void*)gla_seg_state<T, DK, DV, GM>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, GlaStateLds<T, DK, DV>::total);
  return launch_gla<T, DK, DV, GM>(a);
}

#define GLA_CASE(TT, DTC, DKC, DVC)                                                       \
  if (dt == DTC && dk == DKC && dv == DVC) {                                            \
    if constexpr (gla_fits<TT, DKC, DVC>()) {                                            \
      if (query) return GlaLds<TT, DKC, DVC>::total;                                     \
      return a->gate_mode == kGateLogit ? launch_gla_mode<TT, DKC, DVC, kGateLogit>(*a)  \
                                        : launch_gla_mode<TT, DKC, DVC, kGateLogDecay>(*a); \
    }                                                                                    \
    return -1;                                                                           \
  }

int gla_dispatch(int dt, int dk, int dv, const GlaLaunch* a, bool query) {
  if (dt == 1) return gla_dispatch_bf16(dk, dv, a, query);
  GLA_CASE(float, 0, 64, 64)
  GLA_CASE(float, 0, 128, 128)
  return -1;
}

}  // namespace gsa
