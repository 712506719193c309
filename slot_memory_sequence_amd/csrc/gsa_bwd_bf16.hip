// GSA backward on gfx950, bf16 inputs: the chunk form on the matrix cores.
//
// Method: "Gated Slot Attention for Efficient Linear-Time Sequence Modeling",
// Sec. 3.2-3.3 (the function) and App. B (training: the two GLA passes are
// differentiated in reverse order, the write intensity 1 - alpha collects
// the gradient of both, the forget-gate gradient is a reversed cumulative sum
// over tokens, states are recomputed rather than stored); App. A.1 (the chunk
// form: a read of the chunk-start state plus a causal intra-chunk term).
//
// Per chunk of C = 64 tokens, with the chunk-local cumulative decay E (per
// slot), X = (1 - alpha) / E, Z = (1 - alpha) E_C / E, the state W = [Kt | Vt]
// at the chunk start and its adjoint dW at the chunk end:
//   z^T  = E^T * (Wk Q^T  + X^T mask(K Q^T))        pass-1 read        [m x C]
//   ds^T = E^T * (Wv dO^T + X^T mask(V dO^T))       pass-1 read of dO
//   s = softmax(z) (or f(z)),  dz = s (ds - s.ds)  (or f'(z) ds)
//   dq^T = Wk^T (dz*E)^T + K^T mask(X (dz*E)^T)     pass-2 read
//   dk   = Z dWk + mask(X (dz*E)^T)^T Q,  dv = Z dWv + mask(X (s*E)^T)^T dO
//   di   = (1/E) * (E_C dW [k|v]^T + mask(K Q^T)^T (dz*E) + mask(V dO^T)^T (s*E))
//   reverse map of the chunk: [Q | dO]^T [dz*E | s*E]  (what its reads add
//   to the adjoint of its start state); dW at the chunk start =
//   Diag(E_C) dW + that map.
// The gate: with G_t = sum_{r<=t} log alpha_r, dL/dG_t = z dz + s ds - i di
// on the reads and writes of token t, and d log alpha_t = sum_{r>=t} dL/dG_r -
// alpha_t di_t.  The sum over all tokens after a point t0 equals
// <dW_{t0}, W_{t0}> per slot (the adjoint of the state at t0 times that state:
// scaling every later decay by e^eps scales exactly the state carried over
// t0), so each workgroup takes its carry from later chunks from that dot at
// its segment end and sums only inside its own segment.
//
// Launches (one workgroup per (segment, unit); segments of S chunks):
//   1. gsa_bf16_state + gsa_bf16_scan (the forward's): segment start states
//      (skipped when a training forward kept them);
//   2. bwd_bf16_fwd: per segment, chunks in order from its start state: the
//      state carry and the reverse map in MFMA accumulators (state waves),
//      z, ds, s, dz, h = z dz + s ds and dq (pass waves); s, dz, h are kept
//      per token (bf16) for the reverse sweep, the segment's reverse map and
//      decay beside them, and the last segment's end state (every other
//      segment's end state is the next one's start state);
//   3. bwd_bf16_rscan: the end adjoint of every segment (reverse scan of the
//      reverse maps from the final-state gradients) and the initial-state
//      gradients;
//   4. bwd_bf16_rev: per segment, chunks in reverse from its end adjoint:
//      the adjoint update (state waves), dk, dv, di and dg (pass waves).
// A chunk where some slot's decay product falls below 2^-90 (the factorised
// forms divide by E) runs with 16-token sub-chunk reference points
// (chunk_factors; App. A.1's secondary chunking): the intra-chunk terms pass
// between sub-chunks through the decays between their reference points, by
// Horner's rule or by scaling one operand.  Only a chunk in which a 16-token
// sub-chunk decays below 2^-90 runs as an exact token walk of the state waves
// over the fp32 state / adjoint they hold in their accumulators.  128 slots run as two
// groups of 64 (G = 2): a statistics pass of step 2 gives each group's
// softmax statistics, merged into the log-sum-exp and delta that both groups'
// sweeps then take, and the groups' fp32 parts of dq, dk, dv are added last.
#include <type_traits>

#include "../../include/gsa.h"
#include "bf16_common.hpp"
#include "bf16_state.hpp"
#include "common.hpp"
#include "internal.hpp"
#include "launch.hpp"

namespace gsa {
namespace bfb {

using namespace bfk;

// --------------------------------------------------------------- LDS plan
// Shared by both sweeps: the chunk's q, k, v, dO tiles, a bf16 copy of the
// state (forward sweep) or of its adjoint (reverse sweep), one set of chunk
// factors, and two bf16 [C][M] operand tiles (forward sweep: s*E*D and
// dz*E*D for the reverse map, D the decay from the segment start; reverse
// sweep: s*E and dz*E).  The exact path keeps log alpha [C][M] fp32 over X
// and Z, and its reductions in the operand tiles' place.
template <int DK, int DV, int M>
struct BwdLds {
  static constexpr int PAD = 8;
  static constexpr int LDQ = DK + PAD, LDV = DV + PAD, LDW = DK + DV + PAD, LDX = M + PAD, LDE = M + 4;
  static constexpr int oQ = 0;
  static constexpr int oK = oQ + C * LDQ * 2;
  static constexpr int oV = oK + C * LDQ * 2;
  static constexpr int oDo = oV + C * LDV * 2;
  static constexpr int oW = oDo + C * LDV * 2;    // bf16 [M][LDW]
  static constexpr int oX = oW + M * LDW * 2;     // X [C][LDX] bf16 | exact: log alpha [C][M] fp32
  static constexpr int oZ = oX + C * LDX * 2;     // Z [C][LDX] bf16
  static constexpr int oE = oZ + C * LDX * 2;     // E [C][LDE] fp32
  static constexpr int oS = oE + C * LDE * 4;     // s operand [C][LDX] bf16 | exact: reductions
  static constexpr int oDZ = oS + C * LDX * 2;    // dz operand [C][LDX] bf16
  static constexpr int oDec = oDZ + C * LDX * 2;  // chunk decay E_C [M] fp32
  static constexpr int oAux = oDec + M * 4;       // fwd: decay from the segment start [M]; rev: carry [2][M]
  static constexpr int oWt = oAux + 2 * M * 4;    // rev: per pass wave gate sums [4][M] fp32
  static constexpr int oD = oWt + 4 * M * 4;      // decays between reference points [4][M] fp32
  static constexpr int oFlag = oD + 4 * M * 4;    // 2 x NW ints
  static constexpr int total = oFlag + 2 * NW * 4;
  static_assert(C * M * 4 <= 2 * C * LDX * 2, "log alpha fits over X and Z");
  static_assert(2 * 4 * M * 4 <= C * LDX * 2 && 6 * M * 4 <= C * LDE * 4, "exact-path reductions fit");
  static_assert(oK % 16 == 0 && oV % 16 == 0 && oDo % 16 == 0 && oW % 16 == 0 && oX % 16 == 0 &&
                    oZ % 16 == 0 && oE % 16 == 0 && oS % 16 == 0 && oDZ % 16 == 0 && oDec % 16 == 0,
                "LDS tiles must stay 16-byte aligned");
  static_assert(total <= kLdsBytes, "LDS");
};

// Natural log alpha of GPW slots of one token row (the exact path); 0 for a
// row past the end of the sequence.
template <int GPW, class Row>
__device__ __forceinline__ void log_alpha_row(const Row& g, bool valid, float inv_tau, float* dst) {
#pragma unroll
  for (int s = 0; s < GPW; s++) {
    const float x = g.at(s);
    const float la = (fminf(x, 0.f) - log1pf(__expf(-fabsf(x)))) * inv_tau;
    dst[s] = valid ? la : 0.f;
  }
}

// Gate terms of a logit: alpha, 1 - alpha and sigmoid(-g) / tau (hardware
// exp2 / log2; g = +inf gives (1, 0, 0), g = -inf gives (~0, 1, 1/tau)).
__device__ __forceinline__ void gate_terms(float g, float inv_tau, float& a, float& w, float& sn) {
  const float t = g * 1.4426950408889634f;
  const float l2 = fmaxf(-__builtin_amdgcn_logf(1.f + __builtin_amdgcn_exp2f(-t)) * inv_tau, -115.f);
  a = __builtin_amdgcn_exp2f(l2);
  w = 1.f - a;
  sn = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(t)) * inv_tau;
}

// sum over the 16 lanes of a row (DPP quad_perm [1,0,3,2], [2,3,0,1],
// row_half_mirror, row_mirror); every lane of the row gets the same bits
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
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}

__device__ __forceinline__ void store_bf16x4(bf16_t* p, float a, float b, float c, float d) {
  const f32x4 x = {a, b, c, d};
  *reinterpret_cast<bf16x4v*>(p) = pack4(x);
}
__device__ __forceinline__ float4 ld_bf16x4(const bf16_t* p) {
  const uint2 r = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u),
                     __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xffff0000u));
}

// Gradient rows of q, k, v: bf16 for one slot group; fp32 partials when the
// slots run as G > 1 groups (the groups' parts of dq and dk are sums over
// their own slots only and may nearly cancel, so they keep full precision
// until they are added).
template <int G>
using GradT = typename std::conditional<(G > 1), float, bf16_t>::type;
__device__ __forceinline__ void st_grad4(bf16_t* p, const f32x4& v) {
  __builtin_nontemporal_store(__builtin_bit_cast(u32x2, pack4(v)), reinterpret_cast<u32x2*>(p));
}
__device__ __forceinline__ void st_grad4(float* p, const f32x4& v) {
  __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
}
__device__ __forceinline__ void st_grad4(bf16_t* p, float a, float b, float c, float d) { store_bf16x4(p, a, b, c, d); }
__device__ __forceinline__ void st_grad4(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}

// A [C][D] bf16 chunk tile moved as 16-byte vectors by the NTH threads
// 0 .. NTH-1 (the pass waves alone in the forward sweep, so that the state
// waves hold no prefetch registers beside their two accumulator sets).  Rows
// >= rows_valid read the last valid row on load and are written as zeros.
template <int D, int NTH>
struct TileN {
  static constexpr int VPR = D / 8;
  static constexpr int NV = C * VPR / NTH;
  static_assert(NV >= 1 && (C * VPR) % NTH == 0, "tile/thread mismatch");
  uint4 r[NV];
  __device__ __forceinline__ void load(const bf16_t* __restrict__ base, int rows_valid, int tid) {
#pragma unroll
    for (int i = 0; i < NV; i++) {
      const int idx = tid + NTH * i, row = idx / VPR, cv = idx % VPR;
      r[i] = *reinterpret_cast<const uint4*>(base + min(row, rows_valid - 1) * D + cv * 8);
    }
  }
  __device__ __forceinline__ void store(bf16_t* dst, int ld, int rows_valid, int tid) const {
#pragma unroll
    for (int i = 0; i < NV; i++) {
      const int idx = tid + NTH * i, row = idx / VPR, cv = idx % VPR;
      const bool ok = row < rows_valid;
      *reinterpret_cast<uint4*>(dst + row * ld + cv * 8) =
          make_uint4(ok ? r[i].x : 0u, ok ? r[i].y : 0u, ok ? r[i].z : 0u, ok ? r[i].w : 0u);
    }
  }
};

// ======================================================== forward sweep
// Pass waves, first half (before the mid-chunk barrier): token rows 16J ..
// 16J+15.  z and ds, the slot read, dz and h; s, dz and h to the per-token
// workspace (rows < rv); s*E*D and dz*E*D rows to LDS for the reverse map;
// (dz*E)^T as operands for the second half.
// G > 1 (one of G groups of M slots): the softmax read takes each token's
// log-sum-exp over all the slots (lse_rows) and delta = sum over all slots of
// s ds (dl_rows), so s = exp(z - lse) and dz = s (ds - delta).  STATS: only
// the group's own softmax statistics of each token, its log-sum-exp and the
// sum of s ds under its own softmax, to stat_rows[j * 2G + 0 / 1] (the pass
// that the merged lse and delta come from: the same z and ds as the pass that
// takes them, so that dz sums to zero over the slots).
// SUB: the sub-chunk form (chunk_factors): z and ds add the sub-chunks' terms
// by Horner's rule over the decays sD between reference points, the
// reverse-map rows take the decay from the chunk start (the product of the
// rows of sD before this wave's sub-chunk), and the second half gets dz*E in
// fp32 at this wave's reference point (dze) instead of the packed dzb.
template <int DK, int DV, int M, int J, int ACT, int G, bool STATS, bool SUB>
__device__ __forceinline__ void fwd_pass1(int lane, const unsigned char* smem, bf16_t* sS, bf16_t* sDZ,
                                          const float* sSeg, bf16_t* __restrict__ s_rows,
                                          bf16_t* __restrict__ dz_rows, bf16_t* __restrict__ h_rows,
                                          const float* __restrict__ lse_rows, const float* __restrict__ dl_rows,
                                          float* __restrict__ stat_rows, int rv, bf16x8 (&dzb)[M / 32],
                                          f32x4 (&dze)[M / 16]) {
  using Lds = BwdLds<DK, DV, M>;
  constexpr int MT = M / 16, KQ = DK / 32, KV = DV / 32, NP = M / 32;
  constexpr int NR = J + 1, NPR = J / 2 + 1;
  const bf16_t* sQ = reinterpret_cast<const bf16_t*>(smem + Lds::oQ);
  const bf16_t* sK = reinterpret_cast<const bf16_t*>(smem + Lds::oK);
  const bf16_t* sV = reinterpret_cast<const bf16_t*>(smem + Lds::oV);
  const bf16_t* sDo = reinterpret_cast<const bf16_t*>(smem + Lds::oDo);
  const bf16_t* sW = reinterpret_cast<const bf16_t*>(smem + Lds::oW);
  const bf16_t* sX = reinterpret_cast<const bf16_t*>(smem + Lds::oX);
  const float* sE = reinterpret_cast<const float*>(smem + Lds::oE);
  const float* sD = reinterpret_cast<const float*>(smem + Lds::oD);
  const int L = lane & 15, g = lane >> 4;
  const int j = 16 * J + L;

  bf16x8 qf[KQ], df[KV];
#pragma unroll
  for (int s = 0; s < KQ; s++) qf[s] = ld_row(sQ, Lds::LDQ, 16 * J, 32 * s, lane);
#pragma unroll
  for (int s = 0; s < KV; s++) df[s] = ld_row(sDo, Lds::LDV, 16 * J, 32 * s, lane);

  // A^T[r][j] = k_r . q_j, B^T[r][j] = v_r . dO_j for row tiles R <= J (causal)
  f32x4 at[4], bt[4];
#pragma unroll
  for (int R = 0; R < 4; R++) at[R] = bt[R] = zero4();
#pragma unroll
  for (int s = 0; s < KQ; s++)
#pragma unroll
    for (int R = 0; R < NR; R++) at[R] = mma(ld_row(sK, Lds::LDQ, 16 * R, 32 * s, lane), qf[s], at[R]);
#pragma unroll
  for (int s = 0; s < KV; s++)
#pragma unroll
    for (int R = 0; R < NR; R++) bt[R] = mma(ld_row(sV, Lds::LDV, 16 * R, 32 * s, lane), df[s], bt[R]);
#pragma unroll
  for (int i = 0; i < 4; i++)
    if (4 * g + i > L) at[J][i] = bt[J][i] = 0.f;

  // z^T[c][j] = E[j][c] (Wk[c].q_j + sum_r X[r][c] A^T[r][j]); ds^T likewise
  f32x4 z[MT], ds[MT];
#pragma unroll
  for (int ct = 0; ct < MT; ct++) z[ct] = ds[ct] = zero4();
#pragma unroll
  for (int s = 0; s < KQ; s++)
#pragma unroll
    for (int ct = 0; ct < MT; ct++) z[ct] = mma(ld_row(sW, Lds::LDW, 16 * ct, 32 * s, lane), qf[s], z[ct]);
#pragma unroll
  for (int s = 0; s < KV; s++)
#pragma unroll
    for (int ct = 0; ct < MT; ct++)
      ds[ct] = mma(ld_row(sW + DK, Lds::LDW, 16 * ct, 32 * s, lane), df[s], ds[ct]);
  if constexpr (!SUB) {
    bf16x8 af[2], bfr[2];
    af[0] = pack8(at[0], at[1]);
    af[1] = pack8(at[2], at[3]);
    bfr[0] = pack8(bt[0], bt[1]);
    bfr[1] = pack8(bt[2], bt[3]);
#pragma unroll
    for (int pr = 0; pr < NPR; pr++)
#pragma unroll
      for (int ct = 0; ct < MT; ct++) {
        const bf16x8 xa = ld_col(sX, Lds::LDX, 16 * ct, 32 * pr + 4 * g, 32 * pr + 16 + 4 * g, lane);
        z[ct] = mma(xa, af[pr], z[ct]);
        ds[ct] = mma(xa, bfr[pr], ds[ct]);
      }
  } else {
#pragma unroll
    for (int R = 0; R < NR; R++) {
      if (R > 0) {
#pragma unroll
        for (int ct = 0; ct < MT; ct++) {
          const float4 dd = *reinterpret_cast<const float4*>(sD + (R - 1) * M + 16 * ct + 4 * g);
          const float d4[4] = {dd.x, dd.y, dd.z, dd.w};
#pragma unroll
          for (int i = 0; i < 4; i++) {
            z[ct][i] *= d4[i];
            ds[ct][i] *= d4[i];
          }
        }
      }
      const bf16x4v ar = pack4(at[R]), br = pack4(bt[R]);
#pragma unroll
      for (int ct = 0; ct < MT; ct++) {
        const bf16x4v xa = ld_col4(sX, Lds::LDX, 16 * ct, 16 * R + 4 * g, lane);
        z[ct] = mma16(xa, ar, z[ct]);
        ds[ct] = mma16(xa, br, ds[ct]);
      }
    }
  }
  float e[MT][4];
#pragma unroll
  for (int ct = 0; ct < MT; ct++) {
    const float4 ev = *reinterpret_cast<const float4*>(sE + j * Lds::LDE + 16 * ct + 4 * g);
    e[ct][0] = ev.x; e[ct][1] = ev.y; e[ct][2] = ev.z; e[ct][3] = ev.w;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      z[ct][i] *= e[ct][i];
      ds[ct][i] *= e[ct][i];
    }
  }

  // the slot read of token j (over (ct, i) in-lane and the four lane groups)
  f32x4 s[MT], dz[MT];
  if constexpr (ACT == kActSoftmax && G > 1 && !STATS) {
    const bool ok = j < rv;
    const float lj = ok ? lse_rows[j] : 0.f, db = ok ? dl_rows[j] : 0.f;
#pragma unroll
    for (int ct = 0; ct < MT; ct++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        s[ct][i] = __builtin_amdgcn_exp2f((z[ct][i] - lj) * 1.4426950408889634f);
        dz[ct][i] = s[ct][i] * (ds[ct][i] - db);
      }
  } else if constexpr (ACT == kActSoftmax) {
    float mx = z[0][0];
#pragma unroll
    for (int ct = 0; ct < MT; ct++)
#pragma unroll
      for (int i = 0; i < 4; i++) mx = fmaxf(mx, z[ct][i]);
    mx = group4_max(mx);
    float sm = 0.f;
#pragma unroll
    for (int ct = 0; ct < MT; ct++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        s[ct][i] = __builtin_amdgcn_exp2f((z[ct][i] - mx) * 1.4426950408889634f);
        sm += s[ct][i];
      }
    const float smt = group4_sum(sm);
    const float inv = 1.f / smt;
    float db = 0.f;
#pragma unroll
    for (int ct = 0; ct < MT; ct++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        s[ct][i] *= inv;
        db += s[ct][i] * ds[ct][i];
      }
    db = group4_sum(db);
    if constexpr (STATS) {
      if (g == 0 && j < rv) {
        stat_rows[(size_t)j * (2 * G)] = mx + __logf(smt);
        stat_rows[(size_t)j * (2 * G) + 1] = db;
      }
      return;
    }
#pragma unroll
    for (int ct = 0; ct < MT; ct++)
#pragma unroll
      for (int i = 0; i < 4; i++) dz[ct][i] = s[ct][i] * (ds[ct][i] - db);
  } else {
#pragma unroll
    for (int ct = 0; ct < MT; ct++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        s[ct][i] = slot_act<ACT>(z[ct][i]);
        dz[ct][i] = slot_act_grad<ACT>(z[ct][i]) * ds[ct][i];
      }
  }
  const bool valid = j < rv;
#pragma unroll
  for (int ct = 0; ct < MT; ct++) {
    const int c = 16 * ct + 4 * g;
    const float4 dd = *reinterpret_cast<const float4*>(sSeg + c);
    float d4[4] = {dd.x, dd.y, dd.z, dd.w};
    if constexpr (SUB) {  // and the decay from the chunk start to this wave's reference point
#pragma unroll
      for (int r = 0; r < J; r++) {
        const float4 dr = *reinterpret_cast<const float4*>(sD + r * M + c);
        d4[0] *= dr.x;
        d4[1] *= dr.y;
        d4[2] *= dr.z;
        d4[3] *= dr.w;
      }
    }
    float h[4], sed[4], dzed[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      h[i] = z[ct][i] * dz[ct][i] + s[ct][i] * ds[ct][i];
      sed[i] = s[ct][i] * e[ct][i] * d4[i];
      dzed[i] = dz[ct][i] * e[ct][i] * d4[i];
    }
    if (valid) {
      store_bf16x4(s_rows + (size_t)j * M + c, s[ct][0], s[ct][1], s[ct][2], s[ct][3]);
      store_bf16x4(dz_rows + (size_t)j * M + c, dz[ct][0], dz[ct][1], dz[ct][2], dz[ct][3]);
      store_bf16x4(h_rows + (size_t)j * M + c, h[0], h[1], h[2], h[3]);
    }
    store_bf16x4(sS + j * Lds::LDX + c, sed[0], sed[1], sed[2], sed[3]);
    store_bf16x4(sDZ + j * Lds::LDX + c, dzed[0], dzed[1], dzed[2], dzed[3]);
  }
  // (dz*E)^T as B operands over slot pairs (the permuted slot order of pass 2)
  if constexpr (!SUB) {
#pragma unroll
    for (int p = 0; p < NP; p++) {
      const f32x4 a = {dz[2 * p][0] * e[2 * p][0], dz[2 * p][1] * e[2 * p][1], dz[2 * p][2] * e[2 * p][2],
                       dz[2 * p][3] * e[2 * p][3]};
      const f32x4 b = {dz[2 * p + 1][0] * e[2 * p + 1][0], dz[2 * p + 1][1] * e[2 * p + 1][1],
                       dz[2 * p + 1][2] * e[2 * p + 1][2], dz[2 * p + 1][3] * e[2 * p + 1][3]};
      dzb[p] = pack8(a, b);
    }
  } else {
#pragma unroll
    for (int ct = 0; ct < MT; ct++)
#pragma unroll
      for (int i = 0; i < 4; i++) dze[ct][i] = dz[ct][i] * e[ct][i];
  }
}

// Pass waves, second half: dq^T[n][j] = sum_c Wk[c][n] (dz*E)[j][c] +
// sum_{r<=j} K[r][n] A3^T[r][j], A3^T[r][j] = sum_c X[r][c] (dz*E)[j][c].
// SUB: from dze at this wave's reference point, carried back one sub-chunk at
// a time (times sD[R]) before the scores of sub-chunk R; the last set (from
// the chunk start) is the state read's operand.
template <int DK, int DV, int M, int J, int G, bool SUB>
__device__ __forceinline__ void fwd_pass2(int lane, const unsigned char* smem, const bf16x8 (&dzb_in)[M / 32],
                                          const f32x4 (&dze_in)[M / 16], GradT<G>* __restrict__ dq_rows, int rv) {
  using Lds = BwdLds<DK, DV, M>;
  constexpr int NP = M / 32, NKT = DK / 16, MT = M / 16;
  constexpr int NR = J + 1, NPR = J / 2 + 1;
  const bf16_t* sK = reinterpret_cast<const bf16_t*>(smem + Lds::oK);
  const bf16_t* sW = reinterpret_cast<const bf16_t*>(smem + Lds::oW);
  const bf16_t* sX = reinterpret_cast<const bf16_t*>(smem + Lds::oX);
  const float* sD = reinterpret_cast<const float*>(smem + Lds::oD);
  const int L = lane & 15, g = lane >> 4;
  const int j = 16 * J + L;
  f32x4 a3[4];
#pragma unroll
  for (int R = 0; R < 4; R++) a3[R] = zero4();
  bf16x8 dzb[NP];
  if constexpr (!SUB) {
#pragma unroll
    for (int p = 0; p < NP; p++) dzb[p] = dzb_in[p];
#pragma unroll
    for (int p = 0; p < NP; p++)
#pragma unroll
      for (int R = 0; R < NR; R++)
        a3[R] = mma(ld_row2(sX, Lds::LDX, 16 * R, 32 * p + 4 * g, 32 * p + 16 + 4 * g, lane), dzb[p], a3[R]);
  } else {
    f32x4 u[MT];
#pragma unroll
    for (int ct = 0; ct < MT; ct++) u[ct] = dze_in[ct];
#pragma unroll
    for (int R = NR - 1; R >= 0; R--) {
      if (R < J) {
#pragma unroll
        for (int ct = 0; ct < MT; ct++) {
          const float4 dd = *reinterpret_cast<const float4*>(sD + R * M + 16 * ct + 4 * g);
          u[ct][0] *= dd.x;
          u[ct][1] *= dd.y;
          u[ct][2] *= dd.z;
          u[ct][3] *= dd.w;
        }
      }
#pragma unroll
      for (int p = 0; p < NP; p++) dzb[p] = pack8(u[2 * p], u[2 * p + 1]);
#pragma unroll
      for (int p = 0; p < NP; p++)
        a3[R] = mma(ld_row2(sX, Lds::LDX, 16 * R, 32 * p + 4 * g, 32 * p + 16 + 4 * g, lane), dzb[p], a3[R]);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; i++)
    if (4 * g + i > L) a3[J][i] = 0.f;
  bf16x8 a3f[2];
  a3f[0] = pack8(a3[0], a3[1]);
  a3f[1] = pack8(a3[2], a3[3]);
  const bool store = j < rv;
  constexpr int NG = NKT < 4 ? NKT : 4;
#pragma unroll
  for (int n0 = 0; n0 < NKT; n0 += NG) {
    f32x4 acc[NG];
#pragma unroll
    for (int u = 0; u < NG; u++) acc[u] = zero4();
#pragma unroll
    for (int p = 0; p < NP; p++)
#pragma unroll
      for (int u = 0; u < NG; u++)
        acc[u] = mma(ld_col(sW, Lds::LDW, 16 * (n0 + u), 32 * p + 4 * g, 32 * p + 16 + 4 * g, lane), dzb[p],
                     acc[u]);
#pragma unroll
    for (int pr = 0; pr < NPR; pr++)
#pragma unroll
      for (int u = 0; u < NG; u++)
        acc[u] = mma(ld_col(sK, Lds::LDQ, 16 * (n0 + u), 32 * pr + 4 * g, 32 * pr + 16 + 4 * g, lane),
                     a3f[pr], acc[u]);
    if (store) {
#pragma unroll
      for (int u = 0; u < NG; u++)
        st_grad4(dq_rows + (size_t)j * (DK * G) + 16 * (n0 + u) + 4 * g, acc[u]);
    }
  }
}

// Exact forward-sweep chunk (some slot's decay product below the factorised
// range): the state waves walk the tokens on the fp32 state in their
// accumulators (Kt, Vt <- Diag(alpha)(.) + (1 - alpha)[k | v]^T, then the
// reads) and add each token's dq; pass wave 0 takes the slot read of each
// token and writes its reverse-map operand rows (s and dz times the decay
// from the segment start through the token) into the operand tiles, which the
// state waves then contract on the matrix cores as in the factorised path --
// no division by a decay product anywhere.  log alpha of the chunk is in LDS
// (over X, Z), the reductions over E.  Two workgroup barriers per token in
// both halves (fwd_exact_state for the state waves, fwd_exact_pass for the
// others).
template <int DK, int DV, int M, int G, bool STATS>
__device__ __forceinline__ void fwd_exact_state(StateTiles<DK, DV, M, 4>& W, int rv, unsigned char* smem,
                                                GradT<G>* __restrict__ dq_rows, int lane, int sw) {
  using Lds = BwdLds<DK, DV, M>;
  using ST = StateTiles<DK, DV, M, 4>;
  constexpr int MT = M / 16, NCW = ST::NCW;
  const bf16_t* sQ = reinterpret_cast<const bf16_t*>(smem + Lds::oQ);
  const bf16_t* sK = reinterpret_cast<const bf16_t*>(smem + Lds::oK);
  const bf16_t* sV = reinterpret_cast<const bf16_t*>(smem + Lds::oV);
  const bf16_t* sDo = reinterpret_cast<const bf16_t*>(smem + Lds::oDo);
  const float* sLa = reinterpret_cast<const float*>(smem + Lds::oX);
  float* part = reinterpret_cast<float*>(smem + Lds::oE);  // [4][M] scores per state wave
  const float* rDZ = part + 5 * M;                         // [M] dz of the token
  const int L = lane & 15, g = lane >> 4;
  const bool khalf = 16 * (sw * NCW) < DK;  // this wave holds Kt columns (else Vt)
  for (int jt = 0; jt < rv; jt++) {
    float a[MT], w[MT];
#pragma unroll
    for (int ct = 0; ct < MT; ct++) {
      const float la = sLa[jt * M + 16 * ct + L];
      a[ct] = __expf(la);
      w[ct] = -expm1f(la);
    }
    float p[MT];
#pragma unroll
    for (int ct = 0; ct < MT; ct++) p[ct] = 0.f;
#pragma unroll
    for (int n = 0; n < NCW; n++) {
      const int c0 = W.col(sw, n, lane);
      const float4 kv = khalf ? ld_bf16x4(sK + jt * Lds::LDQ + c0) : ld_bf16x4(sV + jt * Lds::LDV + c0 - DK);
      const float4 rd = khalf ? ld_bf16x4(sQ + jt * Lds::LDQ + c0) : ld_bf16x4(sDo + jt * Lds::LDV + c0 - DK);
      const float k4[4] = {kv.x, kv.y, kv.z, kv.w}, q4[4] = {rd.x, rd.y, rd.z, rd.w};
#pragma unroll
      for (int ct = 0; ct < MT; ct++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          W.st[n][ct][i] = a[ct] * W.st[n][ct][i] + w[ct] * k4[i];
          p[ct] += W.st[n][ct][i] * q4[i];
        }
    }
#pragma unroll
    for (int ct = 0; ct < MT; ct++) p[ct] = group4_sum(p[ct]);
    if (g == 0) {
#pragma unroll
      for (int ct = 0; ct < MT; ct++) part[sw * M + 16 * ct + L] = p[ct];
    }
    __syncthreads();  // the token's scores are in LDS
    __syncthreads();  // its read weights are in LDS
    if (!STATS && khalf) {  // dq of token jt over this wave's Kt columns
      float dz[MT];
#pragma unroll
      for (int ct = 0; ct < MT; ct++) dz[ct] = rDZ[16 * ct + L];
#pragma unroll
      for (int n = 0; n < NCW; n++) {
        float x[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
          float acc = 0.f;
#pragma unroll
          for (int ct = 0; ct < MT; ct++) acc += W.st[n][ct][i] * dz[ct];
          x[i] = row_sum16(acc);
        }
        if (L == 0) st_grad4(dq_rows + (size_t)jt * (DK * G) + W.col(sw, n, lane), x[0], x[1], x[2], x[3]);
      }
    }
  }
}

template <int DK, int DV, int M, int ACT, int G, bool STATS>
__device__ __forceinline__ void fwd_exact_pass(int rv, unsigned char* smem, const float* sSeg,
                                               bf16_t* __restrict__ s_rows, bf16_t* __restrict__ dz_rows,
                                               bf16_t* __restrict__ h_rows, const float* __restrict__ lse_rows,
                                               const float* __restrict__ dl_rows, float* __restrict__ stat_rows,
                                               int lane, int wv) {
  using Lds = BwdLds<DK, DV, M>;
  const float* sLa = reinterpret_cast<const float*>(smem + Lds::oX);
  const float* part = reinterpret_cast<const float*>(smem + Lds::oE);
  float* rDZ = reinterpret_cast<float*>(smem + Lds::oE) + 5 * M;
  bf16_t* sS = reinterpret_cast<bf16_t*>(smem + Lds::oS);
  bf16_t* sDZ = reinterpret_cast<bf16_t*>(smem + Lds::oDZ);
  const int tid = wv * 64 + lane;
  // operand rows past the end stay zero (the contraction runs over all C rows)
  for (int e = rv * M + tid; e < C * M; e += 4 * 64) {
    sS[(e / M) * Lds::LDX + e % M] = 0;
    sDZ[(e / M) * Lds::LDX + e % M] = 0;
  }
  const bool on = wv == 0 && lane < M;
  float eseg = on ? sSeg[lane] : 0.f;  // decay from the segment start through the token
  for (int jt = 0; jt < rv; jt++) {
    __syncthreads();  // the token's scores are in LDS
    if (wv == 0) {    // the read of token jt: slot = lane
      const float z = on ? part[lane] + part[M + lane] : 0.f;
      const float ds = on ? part[2 * M + lane] + part[3 * M + lane] : 0.f;
      float s, dz;
      if constexpr (ACT == kActSoftmax && G > 1 && !STATS) {
        s = on ? __expf(z - lse_rows[jt]) : 0.f;
        dz = s * (ds - dl_rows[jt]);
      } else if constexpr (ACT == kActSoftmax) {
        const float mx = wave_max(on ? z : -INFINITY);
        const float e = on ? __expf(z - mx) : 0.f;
        const float smt = sum64(e);
        s = e / smt;
        const float db = sum64(s * ds);
        dz = s * (ds - db);
        if constexpr (STATS) {
          if (lane == 0) {
            stat_rows[(size_t)jt * (2 * G)] = mx + __logf(smt);
            stat_rows[(size_t)jt * (2 * G) + 1] = db;
          }
        }
      } else {
        s = slot_act<ACT>(z);
        dz = slot_act_grad<ACT>(z) * ds;
      }
      if (!STATS && on) {
        eseg *= __expf(sLa[jt * M + lane]);
        rDZ[lane] = dz;
        s_rows[(size_t)jt * M + lane] = f2bf(s);
        dz_rows[(size_t)jt * M + lane] = f2bf(dz);
        h_rows[(size_t)jt * M + lane] = f2bf(z * dz + s * ds);
        sS[jt * Lds::LDX + lane] = f2bf(s * eseg);
        sDZ[jt * Lds::LDX + lane] = f2bf(dz * eseg);
      }
    }
    __syncthreads();  // its read weights are in LDS
  }
}

// One workgroup per (segment, unit).  The state waves and the pass waves run
// separate loops (so that neither holds the other's registers) with the same
// sequence of workgroup barriers: A (chunk staged), M (reverse-map operands
// written), B (chunk done); an exact chunk replaces M by its per-token ones.
// G slot groups (G > 1: unit 2u + h is group h of (b, h) unit u, as in the
// forward's SlotGroups: q, k, v, dO rows of unit u; gate columns hM .. hM +
// M - 1 of g rows of pitch G M; dq rows [rows][G][DK], one partial per group;
// the per-token workspace rows are the group unit's own).
// STATS (with G > 1, the softmax read): the statistics pass of fwd_pass1 only
// (the state carried as usual; no dq, workspace rows, reverse maps or end
// states: the segment start states stay for the pass that follows).
template <int DK, int DV, int M, int ACT, int G, bool STATS>
__global__ void __launch_bounds__(NT, 1)
bwd_bf16_fwd(const bf16_t* __restrict__ qq, const bf16_t* __restrict__ kk, const bf16_t* __restrict__ vv,
             const bf16_t* __restrict__ gg, const bf16_t* __restrict__ dOo, const float* __restrict__ st,
             float* __restrict__ fin, float* __restrict__ rm, float* __restrict__ rdec,
             GradT<G>* __restrict__ dq, bf16_t* __restrict__ s_ws, bf16_t* __restrict__ dz_ws,
             bf16_t* __restrict__ h_ws, int T, int S, int P, float inv_tau, const float* __restrict__ lse,
             const float* __restrict__ delta, float* __restrict__ stats) {
  using Lds = BwdLds<DK, DV, M>;
  using ST = StateTiles<DK, DV, M, 4>;
  constexpr int GPW = M / NW;
  constexpr int NP = M / 32;
  constexpr size_t NE = (size_t)M * (DK + DV);
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  bf16_t* sQ = reinterpret_cast<bf16_t*>(smem + Lds::oQ);
  bf16_t* sK = reinterpret_cast<bf16_t*>(smem + Lds::oK);
  bf16_t* sV = reinterpret_cast<bf16_t*>(smem + Lds::oV);
  bf16_t* sDo = reinterpret_cast<bf16_t*>(smem + Lds::oDo);
  bf16_t* sW = reinterpret_cast<bf16_t*>(smem + Lds::oW);
  bf16_t* sX = reinterpret_cast<bf16_t*>(smem + Lds::oX);
  bf16_t* sZ = reinterpret_cast<bf16_t*>(smem + Lds::oZ);
  float* sE = reinterpret_cast<float*>(smem + Lds::oE);
  bf16_t* sS = reinterpret_cast<bf16_t*>(smem + Lds::oS);
  bf16_t* sDZ = reinterpret_cast<bf16_t*>(smem + Lds::oDZ);
  float* sDec = reinterpret_cast<float*>(smem + Lds::oDec);
  float* sSeg = reinterpret_cast<float*>(smem + Lds::oAux);
  float* sD = reinterpret_cast<float*>(smem + Lds::oD);
  float* sLa = reinterpret_cast<float*>(smem + Lds::oX);
  int* sFlag = reinterpret_cast<int*>(smem + Lds::oFlag);

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const bool is_state = wv >= 4;
  const int sw = wv - 4;
  const int slot0 = wv * GPW;
  const int seg = blockIdx.x % P, unit = blockIdx.x / P;
  const int nchunks = (T + C - 1) / C;
  const int c_begin = seg * S, c_end = min(c_begin + S, nchunks);
  constexpr int GS = M * G;                                 // gate row pitch
  const int grp = unit % G;
  const size_t ub = (size_t)(unit / G) * T, wb = (size_t)unit * T;  // token rows, workspace rows
  const bf16_t* qb = qq + ub * DK;
  const bf16_t* kb = kk + ub * DK;
  const bf16_t* vb = vv + ub * DV;
  const bf16_t* db = dOo + ub * DV;
  const bf16_t* gb = gg + ub * GS + grp * M + slot0;
  GradT<G>* dqb = dq + (ub * G + grp) * DK;
  const float* stp = st + ((size_t)unit * P + seg) * NE;
  float* rmp = rm + ((size_t)unit * P + seg) * NE;
  auto rows_of = [&](int ch) { return min(C, T - ch * C); };

  typedef GateRow<GPW> Row;
  Row gr;
  // the chunk tiles go through the pass waves' registers only (threads 0 .. 255)
  TileN<DK, 256> pq, pk;
  TileN<DV, 256> pv, pd;
  auto load_tiles = [&](int ch, int tid_) {
    const int t0 = ch * C, rv = rows_of(ch);
    pq.load(qb + (size_t)t0 * DK, rv, tid_);
    pk.load(kb + (size_t)t0 * DK, rv, tid_);
    pv.load(vb + (size_t)t0 * DV, rv, tid_);
    pd.load(db + (size_t)t0 * DV, rv, tid_);
  };
  auto load_gates = [&](int ch, int lane_) {
    gr.load(gb + (size_t)(ch * C + min(lane_, rows_of(ch) - 1)) * GS);
  };
  // stage chunk ch (the pass waves its tiles, every wave its factors),
  // barrier A, log alpha for an exact chunk, the loads of the next chunk
  // (this one again at the end); returns the chunk's regime bits
  auto stage = [&](auto pass, int ch, int it, int lane_, int tid_) -> int {
    const int rv = rows_of(ch);
    if constexpr (decltype(pass)::value) {
      pq.store(sQ, Lds::LDQ, rv, tid_);
      pk.store(sK, Lds::LDQ, rv, tid_);
      pv.store(sV, Lds::LDV, rv, tid_);
      pd.store(sDo, Lds::LDV, rv, tid_);
    }
    gr.pin();
    float E[GPW];
    const int small = chunk_factors<GPW, Lds::LDX, Lds::LDE, M>(gr, lane_ < rv, inv_tau, lane_, slot0, sX, sZ,
                                                                 sE, sD, sDec, E);
    const int regime = block_or(small, sFlag, it, lane_, wv);
    if (regime & kNeedExact) {  // every factor reader is past barrier A
      float la[GPW];
      log_alpha_row<GPW>(gr, lane_ < rv, inv_tau, la);
      store_f32_row<GPW>(sLa + lane_ * M + slot0, la);
    }
    const int cn = min(ch + 1, c_end - 1);
    load_gates(cn, lane_);
    if constexpr (decltype(pass)::value) load_tiles(cn, tid_);
    return regime;
  };
  using Pass = std::integral_constant<bool, true>;
  using State = std::integral_constant<bool, false>;

  load_gates(c_begin, lane);
  if (tid < M) sSeg[tid] = 1.f;
  if (is_state) {
    ST W, R;
    W.load_w(stp, sw, lane);
    R.zero();
    for (int ch = c_begin; ch < c_end; ch++) {
      int lane_i = lane, tid_i = tid;
      asm volatile("" : "+v"(lane_i), "+v"(tid_i));
      const int rv = rows_of(ch);
      W.store_copy(sW, Lds::LDW, sw, lane_i);  // the chunk's start state for the pass waves
      const bool slow = stage(State{}, ch, ch - c_begin, lane_i, tid_i) & kNeedExact;
      if (!slow) {
        W.carry(sK, Lds::LDQ, sV, Lds::LDV, sZ, Lds::LDX, sDec, sw, lane_i);
        __syncthreads();  // M: the reverse-map operands are in LDS
      } else {
        __syncthreads();  // log alpha is in LDS
        fwd_exact_state<DK, DV, M, G, STATS>(W, rv, smem, dqb + (size_t)ch * C * (DK * G), lane_i, sw);
      }
      // the chunk's reverse map (operand rows from the passes or the walk)
      if constexpr (!STATS) R.update2(sQ, Lds::LDQ, sDo, Lds::LDV, sDZ, sS, Lds::LDX, nullptr, sw, lane_i);
      __syncthreads();  // B: every reader of this chunk's tiles, factors and copies is done
    }
    // the segment's reverse map; the last segment's end state (the final
    // state: every other segment's end state is the next one's start state,
    // which st already holds)
    if constexpr (!STATS) {
      if (seg == P - 1) W.store_w(fin + (size_t)unit * NE, sw, lane);
      R.store_w(rmp, sw, lane);
    }
  } else {
    load_tiles(c_begin, tid);
    bf16x8 dzb[NP];
    for (int ch = c_begin; ch < c_end; ch++) {
      f32x4 dze[M / 16];  // dz*E of the sub-chunk form (both halves before M)
      int lane_i = lane, tid_i = tid;
      asm volatile("" : "+v"(lane_i), "+v"(tid_i));
      const int t0 = ch * C, rv = rows_of(ch);
      const int regime = stage(Pass{}, ch, ch - c_begin, lane_i, tid_i);
      const bool slow = regime & kNeedExact, sub = regime & kNeedSub;
      bf16_t* srow = s_ws + (wb + t0) * M;
      bf16_t* dzrow = dz_ws + (wb + t0) * M;
      bf16_t* hrow = h_ws + (wb + t0) * M;
      const float* lrow = G > 1 && !STATS ? lse + ub + t0 : nullptr;
      const float* drow = G > 1 && !STATS ? delta + ub + t0 : nullptr;
      float* strow = STATS ? stats + ((ub + t0) * G + grp) * 2 : nullptr;
      if (!slow) {
#define GSA_FWD_PASS1(JJ, SB)                                                                            \
  fwd_pass1<DK, DV, M, JJ, ACT, G, STATS, SB>(lane_i, smem, sS, sDZ, sSeg, srow, dzrow, hrow, lrow, drow, \
                                              strow, rv, dzb, dze)
        if (!sub) {
          switch (wv) {
            case 0: GSA_FWD_PASS1(0, false); break;
            case 1: GSA_FWD_PASS1(1, false); break;
            case 2: GSA_FWD_PASS1(2, false); break;
            default: GSA_FWD_PASS1(3, false); break;
          }
        } else {
          // some slot decays out of the chunk form's range: sub-chunk
          // reference points; both halves before M (dz*E stays in this
          // branch's registers)
          GradT<G>* dqrow = dqb + (size_t)t0 * (DK * G);
#define GSA_FWD_SUB(JJ)                                                          \
  GSA_FWD_PASS1(JJ, true);                                                       \
  if constexpr (!STATS) fwd_pass2<DK, DV, M, JJ, G, true>(lane_i, smem, dzb, dze, dqrow, rv)
          switch (wv) {
            // rows of sub-chunk 0: its reference point is the chunk start, so
            // the sub-chunk form is the plain one (pass 2 after M as usual)
            case 0: GSA_FWD_PASS1(0, false); break;
            case 1: GSA_FWD_SUB(1); break;
            case 2: GSA_FWD_SUB(2); break;
            default: GSA_FWD_SUB(3); break;
          }
#undef GSA_FWD_SUB
        }
#undef GSA_FWD_PASS1
        __syncthreads();  // M
        // the decay from the segment start, advanced past this chunk (its
        // readers are all before M; E_C is rewritten only after B)
        if (tid_i < M) sSeg[tid_i] *= sDec[tid_i];
        GradT<G>* dqrow = dqb + (size_t)t0 * (DK * G);
        if constexpr (!STATS) {
          if (!sub || wv == 0) {
            switch (wv) {
              case 0: fwd_pass2<DK, DV, M, 0, G, false>(lane_i, smem, dzb, dze, dqrow, rv); break;
              case 1: fwd_pass2<DK, DV, M, 1, G, false>(lane_i, smem, dzb, dze, dqrow, rv); break;
              case 2: fwd_pass2<DK, DV, M, 2, G, false>(lane_i, smem, dzb, dze, dqrow, rv); break;
              default: fwd_pass2<DK, DV, M, 3, G, false>(lane_i, smem, dzb, dze, dqrow, rv); break;
            }
          }
        }
      } else {
        __syncthreads();  // log alpha is in LDS
        fwd_exact_pass<DK, DV, M, ACT, G, STATS>(rv, smem, sSeg, srow, dzrow, hrow, lrow, drow, strow, lane_i, wv);
        if (tid_i < M) sSeg[tid_i] *= sDec[tid_i];  // read by the walk before its first barrier
      }
      __syncthreads();  // B
    }
  }
  __syncthreads();
  if (!STATS && tid < M) rdec[((size_t)unit * P + seg) * M + tid] = sSeg[tid];
}

// ======================================================== reverse scan
// One thread per (unit, four consecutive elements of a slot row), serial
// over the segments from the last: slot p of rm holds segment p's reverse map
// on entry and on exit the adjoint of the state at segment p's end (from the
// tokens after it and the final-state gradients dkf / dvf, nullable = zero);
// what is carried out of segment 0 is the gradient of the initial states.
template <int DK, int DV, int M>
__global__ void __launch_bounds__(256)
bwd_bf16_rscan(float* __restrict__ rm, const float* __restrict__ rdec, const float* __restrict__ dkf,
               const float* __restrict__ dvf, float* __restrict__ dk0, float* __restrict__ dv0, int units,
               int P) {
  constexpr int NE = M * (DK + DV), BATCH = 8;
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long long)units * (NE / 4)) return;
  const int unit = (int)(gid / (NE / 4)), e = 4 * (int)(gid % (NE / 4));
  const int c = e / (DK + DV), cl = e % (DK + DV);
  const size_t ko = ((size_t)unit * M + c) * DK + cl, vo = ((size_t)unit * M + c) * DV + cl - DK;
  f32x4 W = zero4();
  if (cl < DK) {
    if (dkf) W = *reinterpret_cast<const f32x4*>(dkf + ko);
  } else {
    if (dvf) W = *reinterpret_cast<const f32x4*>(dvf + vo);
  }
  f32x4* sl = reinterpret_cast<f32x4*>(rm + (size_t)unit * P * NE + e);
  const float* dc = rdec + (size_t)unit * P * M + c;
  for (int n0 = 0; n0 < P; n0 += BATCH) {
    f32x4 x[BATCH];
    float d[BATCH];
#pragma unroll
    for (int i = 0; i < BATCH; i++) {
      if (n0 + i < P) {
        const int p = P - 1 - (n0 + i);
        x[i] = sl[(size_t)p * (NE / 4)];
        d[i] = dc[(size_t)p * M];
      }
    }
#pragma unroll
    for (int i = 0; i < BATCH; i++) {
      if (n0 + i < P) {
        const int p = P - 1 - (n0 + i);
        sl[(size_t)p * (NE / 4)] = W;
        W = d[i] * W + x[i];
      }
    }
  }
  if (cl < DK) {
    if (dk0) *reinterpret_cast<f32x4*>(dk0 + ko) = W;
  } else {
    if (dv0) *reinterpret_cast<f32x4*>(dv0 + vo) = W;
  }
}

// ======================================================== reverse sweep
// Pass waves: write-token rows j = 16J .. 16J+15 of the chunk, from the bf16
// copy of the adjoint at the chunk end.  dk and dv rows are written; di and
// the gate terms give each (token, slot) its part of d log alpha: the sum
// over the wave's rows from j on (pre), the wave's total per slot (sWt[J]).
// The rest (later waves' totals and the carry from later chunks) is added
// after the next barrier by rev_pass_finish.
// SUB: the sub-chunk form (chunk_factors; s*E and dz*E staged at each token's
// own reference point): the X rows of this wave are carried to the reference
// point of each later read sub-chunk T (times sD[J] ... sD[T-1]) before its
// scores, and di adds the read sub-chunks' terms by Horner's rule from the
// chunk end (the adjoint term first, times sD[3], then each sub-chunk T = 3 ..
// J after a scaling by sD[T]).
template <int DK, int DV, int M, int J, int G, bool SUB>
__device__ __forceinline__ void rev_pass(int lane, const unsigned char* smem, float* sWt,
                                         const bf16_t* __restrict__ h_rows, const bf16_t* __restrict__ g_rows,
                                         GradT<G>* __restrict__ dk_rows, GradT<G>* __restrict__ dv_rows, int rv,
                                         float inv_tau, float (&pre)[M / 16][4], float (&sn)[M / 16][4]) {
  using Lds = BwdLds<DK, DV, M>;
  constexpr int MT = M / 16, KQ = DK / 32, KV = DV / 32, NP = M / 32, NKT = DK / 16, NVT = DV / 16;
  constexpr int PR0 = J / 2;  // first read-row tile pair at or after this wave's rows
  const bf16_t* sQ = reinterpret_cast<const bf16_t*>(smem + Lds::oQ);
  const bf16_t* sK = reinterpret_cast<const bf16_t*>(smem + Lds::oK);
  const bf16_t* sV = reinterpret_cast<const bf16_t*>(smem + Lds::oV);
  const bf16_t* sDo = reinterpret_cast<const bf16_t*>(smem + Lds::oDo);
  const bf16_t* sW = reinterpret_cast<const bf16_t*>(smem + Lds::oW);
  const bf16_t* sX = reinterpret_cast<const bf16_t*>(smem + Lds::oX);
  const bf16_t* sZ = reinterpret_cast<const bf16_t*>(smem + Lds::oZ);
  const float* sE = reinterpret_cast<const float*>(smem + Lds::oE);
  const bf16_t* sS = reinterpret_cast<const bf16_t*>(smem + Lds::oS);
  const bf16_t* sDZ = reinterpret_cast<const bf16_t*>(smem + Lds::oDZ);
  const float* sDec = reinterpret_cast<const float*>(smem + Lds::oDec);
  const float* sD = reinterpret_cast<const float*>(smem + Lds::oD);
  const int L = lane & 15, g = lane >> 4;
  const int j = 16 * J + L;
  const bool valid = j < rv;
  const int jr = valid ? j : rv - 1;  // rows past the end read the last valid row (masked below)

  // this lane's h and gate logits (token j, slots 16ct + 4g + 0..3), issued first
  float4 hv[MT], gv[MT];
#pragma unroll
  for (int ct = 0; ct < MT; ct++) {
    hv[ct] = ld_bf16x4(h_rows + (size_t)jr * M + 16 * ct + 4 * g);
    gv[ct] = ld_bf16x4(g_rows + (size_t)jr * (M * G) + 16 * ct + 4 * g);
  }

  bf16x8 kf[KQ], vf[KV];
#pragma unroll
  for (int s = 0; s < KQ; s++) kf[s] = ld_row(sK, Lds::LDQ, 16 * J, 32 * s, lane);
#pragma unroll
  for (int s = 0; s < KV; s++) vf[s] = ld_row(sV, Lds::LDV, 16 * J, 32 * s, lane);

  // S1[t'][j] = q_t' . k_j, S2[t'][j] = dO_t' . v_j for read rows t' >= j
  f32x4 s1[4], s2[4];
#pragma unroll
  for (int T = 0; T < 4; T++) s1[T] = s2[T] = zero4();
#pragma unroll
  for (int s = 0; s < KQ; s++)
#pragma unroll
    for (int T = J; T < 4; T++) s1[T] = mma(ld_row(sQ, Lds::LDQ, 16 * T, 32 * s, lane), kf[s], s1[T]);
#pragma unroll
  for (int s = 0; s < KV; s++)
#pragma unroll
    for (int T = J; T < 4; T++) s2[T] = mma(ld_row(sDo, Lds::LDV, 16 * T, 32 * s, lane), vf[s], s2[T]);
  // A_dq[t'][j] = sum_c dzE[t'][c] X[j][c], A2[t'][j] = sum_c sE[t'][c] X[j][c]
  bf16x8 xb[NP];
#pragma unroll
  for (int p = 0; p < NP; p++) xb[p] = ld_row2(sX, Lds::LDX, 16 * J, 32 * p + 4 * g, 32 * p + 16 + 4 * g, lane);
  f32x4 ad[4], a2[4];
#pragma unroll
  for (int T = 0; T < 4; T++) ad[T] = a2[T] = zero4();
  if constexpr (!SUB) {
#pragma unroll
    for (int p = 0; p < NP; p++)
#pragma unroll
      for (int T = J; T < 4; T++) {
        ad[T] = mma(ld_row2(sDZ, Lds::LDX, 16 * T, 32 * p + 4 * g, 32 * p + 16 + 4 * g, lane), xb[p], ad[T]);
        a2[T] = mma(ld_row2(sS, Lds::LDX, 16 * T, 32 * p + 4 * g, 32 * p + 16 + 4 * g, lane), xb[p], a2[T]);
      }
  } else {
    // X of this lane's row j (slots 32p + 4g + 0..3 and 32p + 16 + 4g + 0..3)
    // carried to read sub-chunk T: times sD[J] ... sD[T-1], formed per T from
    // the bf16 row (no fp32 copy held across the sub-chunks)
#pragma unroll
    for (int T = J; T < 4; T++) {
#pragma unroll
      for (int p = 0; p < NP; p++) {
        bf16x8 xt = xb[p];
        if (T > J) {
          f32x8 xr = __builtin_convertvector(xb[p], f32x8);
#pragma unroll
          for (int r = J; r < T; r++) {
            const float4 lo = *reinterpret_cast<const float4*>(sD + r * M + 32 * p + 4 * g);
            const float4 hi = *reinterpret_cast<const float4*>(sD + r * M + 32 * p + 16 + 4 * g);
            xr[0] *= lo.x; xr[1] *= lo.y; xr[2] *= lo.z; xr[3] *= lo.w;
            xr[4] *= hi.x; xr[5] *= hi.y; xr[6] *= hi.z; xr[7] *= hi.w;
          }
          xt = __builtin_convertvector(xr, bf16x8);
        }
        ad[T] = mma(ld_row2(sDZ, Lds::LDX, 16 * T, 32 * p + 4 * g, 32 * p + 16 + 4 * g, lane), xt, ad[T]);
        a2[T] = mma(ld_row2(sS, Lds::LDX, 16 * T, 32 * p + 4 * g, 32 * p + 16 + 4 * g, lane), xt, a2[T]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; i++)
    if (4 * g + i < L) s1[J][i] = s2[J][i] = ad[J][i] = a2[J][i] = 0.f;  // causal: t' >= j
  bf16x8 s1f[2], s2f[2], adf[2], a2f[2];
#pragma unroll
  for (int pr = 0; pr < 2; pr++) {
    s1f[pr] = pack8(s1[2 * pr], s1[2 * pr + 1]);
    s2f[pr] = pack8(s2[2 * pr], s2[2 * pr + 1]);
    adf[pr] = pack8(ad[2 * pr], ad[2 * pr + 1]);
    a2f[pr] = pack8(a2[2 * pr], a2[2 * pr + 1]);
  }

  // dk^T[n][j] = sum_c dWk[c][n] Z[j][c] + sum_t' Q[t'][n] A_dq[t'][j]; dv^T likewise
  bf16x8 zb[NP];
#pragma unroll
  for (int p = 0; p < NP; p++) zb[p] = ld_row2(sZ, Lds::LDX, 16 * J, 32 * p + 4 * g, 32 * p + 16 + 4 * g, lane);
  constexpr int NG = 4;
  static_assert(NKT % NG == 0 && NVT % NG == 0, "column groups");
#pragma unroll
  for (int n0 = 0; n0 < NKT + NVT; n0 += NG) {
    const bool kpart = n0 < NKT;
    const int nb = kpart ? n0 : n0 - NKT;
    f32x4 acc[NG];
#pragma unroll
    for (int u = 0; u < NG; u++) acc[u] = zero4();
#pragma unroll
    for (int p = 0; p < NP; p++)
#pragma unroll
      for (int u = 0; u < NG; u++)
        acc[u] = mma(ld_col(sW + (kpart ? 0 : DK), Lds::LDW, 16 * (nb + u), 32 * p + 4 * g, 32 * p + 16 + 4 * g,
                            lane),
                     zb[p], acc[u]);
#pragma unroll
    for (int pr = PR0; pr < 2; pr++)
#pragma unroll
      for (int u = 0; u < NG; u++)
        acc[u] = kpart ? mma(ld_col(sQ, Lds::LDQ, 16 * (nb + u), 32 * pr + 4 * g, 32 * pr + 16 + 4 * g, lane),
                             adf[pr], acc[u])
                       : mma(ld_col(sDo, Lds::LDV, 16 * (nb + u), 32 * pr + 4 * g, 32 * pr + 16 + 4 * g, lane),
                             a2f[pr], acc[u]);
    if (valid) {
#pragma unroll
      for (int u = 0; u < NG; u++) {
        GradT<G>* dst = kpart ? dk_rows + (size_t)j * (DK * G) : dv_rows + (size_t)j * (DV * G);
        st_grad4(dst + 16 * (nb + u) + 4 * g, acc[u]);
      }
    }
  }

  // di^T[c][j] = (E_C[c] sum_n dW[c][n] [k|v]_j[n] + sum_t' (dzE[t'][c] S1[t'][j] +
  // sE[t'][c] S2[t'][j])) / E[j][c]
  f32x4 di[MT];
#pragma unroll
  for (int ct = 0; ct < MT; ct++) di[ct] = zero4();
#pragma unroll
  for (int s = 0; s < KQ; s++)
#pragma unroll
    for (int ct = 0; ct < MT; ct++) di[ct] = mma(ld_row(sW, Lds::LDW, 16 * ct, 32 * s, lane), kf[s], di[ct]);
#pragma unroll
  for (int s = 0; s < KV; s++)
#pragma unroll
    for (int ct = 0; ct < MT; ct++)
      di[ct] = mma(ld_row(sW + DK, Lds::LDW, 16 * ct, 32 * s, lane), vf[s], di[ct]);
  if constexpr (!SUB) {
#pragma unroll
    for (int ct = 0; ct < MT; ct++) {
      const float4 d = *reinterpret_cast<const float4*>(sDec + 16 * ct + 4 * g);
      di[ct][0] *= d.x;
      di[ct][1] *= d.y;
      di[ct][2] *= d.z;
      di[ct][3] *= d.w;
    }
#pragma unroll
    for (int pr = PR0; pr < 2; pr++)
#pragma unroll
      for (int ct = 0; ct < MT; ct++) {
        di[ct] = mma(ld_col(sDZ, Lds::LDX, 16 * ct, 32 * pr + 4 * g, 32 * pr + 16 + 4 * g, lane), s1f[pr], di[ct]);
        di[ct] = mma(ld_col(sS, Lds::LDX, 16 * ct, 32 * pr + 4 * g, 32 * pr + 16 + 4 * g, lane), s2f[pr], di[ct]);
      }
  } else {
#pragma unroll
    for (int T = 3; T >= J; T--) {
#pragma unroll
      for (int ct = 0; ct < MT; ct++) {
        const float4 d = *reinterpret_cast<const float4*>(sD + T * M + 16 * ct + 4 * g);
        di[ct][0] *= d.x;
        di[ct][1] *= d.y;
        di[ct][2] *= d.z;
        di[ct][3] *= d.w;
      }
      const bf16x4v b1 = pack4(s1[T]), b2 = pack4(s2[T]);
#pragma unroll
      for (int ct = 0; ct < MT; ct++) {
        di[ct] = mma16(ld_col4(sDZ, Lds::LDX, 16 * ct, 16 * T + 4 * g, lane), b1, di[ct]);
        di[ct] = mma16(ld_col4(sS, Lds::LDX, 16 * ct, 16 * T + 4 * g, lane), b2, di[ct]);
      }
    }
  }

  // gate: u = h - (1 - alpha) di; sums over the wave's rows from j on (DPP
  // row shifts towards lower lanes), pre = that sum - alpha di
#pragma unroll
  for (int ct = 0; ct < MT; ct++) {
    const float4 e = *reinterpret_cast<const float4*>(sE + j * Lds::LDE + 16 * ct + 4 * g);
    const float ev[4] = {e.x, e.y, e.z, e.w};
    const float hh[4] = {hv[ct].x, hv[ct].y, hv[ct].z, hv[ct].w};
    const float gl[4] = {gv[ct].x, gv[ct].y, gv[ct].z, gv[ct].w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const float d = di[ct][i] * __builtin_amdgcn_rcpf(ev[i]);
      float a, w;
      gate_terms(gl[i], inv_tau, a, w, sn[ct][i]);
      float x = valid ? hh[i] - w * d : 0.f;
      x += dpp_zero<0x101, 0xf>(x);  // row_shl:1
      x += dpp_zero<0x102, 0xf>(x);  // row_shl:2
      x += dpp_zero<0x104, 0xf>(x);  // row_shl:4
      x += dpp_zero<0x108, 0xf>(x);  // row_shl:8
      pre[ct][i] = x - a * d;
      if (L == 0) sWt[J * M + 16 * ct + 4 * g + i] = x;
    }
  }
}

// After the barrier that publishes every wave's totals: d log alpha = pre +
// the totals of the later waves of this chunk + the carry from later chunks;
// dg = that * sigmoid(-g) / tau.
template <int M, int J, int G>
__device__ __forceinline__ void rev_pass_finish(int lane, const float* sWt, const float* carry,
                                                bf16_t* __restrict__ dg_rows, int rv,
                                                const float (&pre)[M / 16][4], const float (&sn)[M / 16][4]) {
  constexpr int MT = M / 16;
  const int L = lane & 15, g = lane >> 4, j = 16 * J + L;
#pragma unroll
  for (int ct = 0; ct < MT; ct++) {
    const int c = 16 * ct + 4 * g;
    float4 add = *reinterpret_cast<const float4*>(carry + c);
#pragma unroll
    for (int J2 = J + 1; J2 < 4; J2++) {
      const float4 t = *reinterpret_cast<const float4*>(sWt + J2 * M + c);
      add.x += t.x; add.y += t.y; add.z += t.z; add.w += t.w;
    }
    if (j < rv)
      store_bf16x4(dg_rows + (size_t)j * (M * G) + c, (pre[ct][0] + add.x) * sn[ct][0], (pre[ct][1] + add.y) * sn[ct][1],
                   (pre[ct][2] + add.z) * sn[ct][2], (pre[ct][3] + add.w) * sn[ct][3]);
  }
}

// Exact reverse-sweep chunk: the state waves walk the tokens backwards on the
// fp32 adjoint in their accumulators (dW += [dz q^T | s dO^T] of the token,
// dk, dv and di from it, then dW *= alpha), pass wave 0 forms each token's
// gate gradient; s, dz and h come unscaled from the per-token workspace.  On
// return the state waves' accumulators hold the adjoint at the chunk start
// and sWt[0] the chunk's total of the gate terms (sWt[1..3] = 0).  One
// workgroup barrier per token in both halves.
template <int DK, int DV, int M, int G>
__device__ __forceinline__ void rev_exact_state(StateTiles<DK, DV, M, 4>& W, int rv, unsigned char* smem,
                                                const bf16_t* __restrict__ s_rows,
                                                const bf16_t* __restrict__ dz_rows, GradT<G>* __restrict__ dk_rows,
                                                GradT<G>* __restrict__ dv_rows, int lane, int sw) {
  using Lds = BwdLds<DK, DV, M>;
  using ST = StateTiles<DK, DV, M, 4>;
  constexpr int MT = M / 16, NCW = ST::NCW;
  const bf16_t* sQ = reinterpret_cast<const bf16_t*>(smem + Lds::oQ);
  const bf16_t* sK = reinterpret_cast<const bf16_t*>(smem + Lds::oK);
  const bf16_t* sV = reinterpret_cast<const bf16_t*>(smem + Lds::oV);
  const bf16_t* sDo = reinterpret_cast<const bf16_t*>(smem + Lds::oDo);
  const float* sLa = reinterpret_cast<const float*>(smem + Lds::oX);
  float* dpart = reinterpret_cast<float*>(smem + Lds::oS);  // [2][4][M]: di partials per state wave
  const int L = lane & 15, g = lane >> 4;
  const bool khalf = 16 * (sw * NCW) < DK;
  for (int jt = rv - 1, n = 0; jt >= 0; jt--, n++) {
    float* dp = dpart + (n & 1) * 4 * M;
    float a[MT], w[MT], rd[MT];
#pragma unroll
    for (int ct = 0; ct < MT; ct++) {
      const float la = sLa[jt * M + 16 * ct + L];
      a[ct] = __expf(la);
      w[ct] = -expm1f(la);
      rd[ct] = bf2f(khalf ? dz_rows[(size_t)jt * M + 16 * ct + L] : s_rows[(size_t)jt * M + 16 * ct + L]);
    }
    float p[MT];
#pragma unroll
    for (int ct = 0; ct < MT; ct++) p[ct] = 0.f;
#pragma unroll
    for (int n2 = 0; n2 < NCW; n2++) {
      const int c0 = W.col(sw, n2, lane);
      const float4 kv = khalf ? ld_bf16x4(sK + jt * Lds::LDQ + c0) : ld_bf16x4(sV + jt * Lds::LDV + c0 - DK);
      const float4 qv = khalf ? ld_bf16x4(sQ + jt * Lds::LDQ + c0) : ld_bf16x4(sDo + jt * Lds::LDV + c0 - DK);
      const float k4[4] = {kv.x, kv.y, kv.z, kv.w}, q4[4] = {qv.x, qv.y, qv.z, qv.w};
      float x[4];
#pragma unroll
      for (int i = 0; i < 4; i++) {
        float acc = 0.f;
#pragma unroll
        for (int ct = 0; ct < MT; ct++) {
          W.st[n2][ct][i] += rd[ct] * q4[i];
          acc += w[ct] * W.st[n2][ct][i];
          p[ct] += W.st[n2][ct][i] * k4[i];
        }
        x[i] = row_sum16(acc);
      }
      if (L == 0) {
        GradT<G>* dst = khalf ? dk_rows + (size_t)jt * (DK * G) + c0 : dv_rows + (size_t)jt * (DV * G) + c0 - DK;
        st_grad4(dst, x[0], x[1], x[2], x[3]);
      }
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int ct = 0; ct < MT; ct++) W.st[n2][ct][i] *= a[ct];
    }
#pragma unroll
    for (int ct = 0; ct < MT; ct++) p[ct] = group4_sum(p[ct]);
    if (g == 0) {
#pragma unroll
      for (int ct = 0; ct < MT; ct++) dp[sw * M + 16 * ct + L] = p[ct];
    }
    __syncthreads();  // the token's di partials are in LDS
  }
}

template <int M, int G>
__device__ __forceinline__ void rev_exact_pass(int rv, const unsigned char* smem, int oS, const float* carry,
                                               float* sWt, const bf16_t* __restrict__ h_rows,
                                               const bf16_t* __restrict__ g_rows, bf16_t* __restrict__ dg_rows,
                                               float inv_tau, int lane, int wv) {
  const float* dpart = reinterpret_cast<const float*>(smem + oS);
  float run = 0.f;  // wave 0: the sum of the gate terms of the chunk's tokens from jt on
  for (int jt = rv - 1, n = 0; jt >= 0; jt--, n++) {
    __syncthreads();  // the token's di partials are in LDS
    if (wv == 0 && lane < M) {
      const float* dp = dpart + (n & 1) * 4 * M;
      const float d = dp[lane] + dp[M + lane] + dp[2 * M + lane] + dp[3 * M + lane];
      float a, w, sn;
      gate_terms(bf2f(g_rows[(size_t)jt * (M * G) + lane]), inv_tau, a, w, sn);
      run += bf2f(h_rows[(size_t)jt * M + lane]) - w * d;
      dg_rows[(size_t)jt * (M * G) + lane] = f2bf((run + carry[lane] - a * d) * sn);
    }
  }
  if (wv == 0 && lane < M) {
    sWt[lane] = run;
    sWt[M + lane] = sWt[2 * M + lane] = sWt[3 * M + lane] = 0.f;
  }
}

// One workgroup per (segment, unit), chunks from the segment's end.  As in the
// forward sweep the two roles run separate loops with the same barriers: A
// (chunk staged), B (chunk done, its gate totals published); an exact chunk
// adds one barrier per token.
template <int DK, int DV, int M, int G>
__global__ void __launch_bounds__(NT, 1)
bwd_bf16_rev(const bf16_t* __restrict__ qq, const bf16_t* __restrict__ kk, const bf16_t* __restrict__ vv,
             const bf16_t* __restrict__ gg, const bf16_t* __restrict__ dOo, const float* __restrict__ st,
             const float* __restrict__ fin, const float* __restrict__ rm, const bf16_t* __restrict__ s_ws,
             const bf16_t* __restrict__ dz_ws, const bf16_t* __restrict__ h_ws, GradT<G>* __restrict__ dk,
             GradT<G>* __restrict__ dv, bf16_t* __restrict__ dg, int T, int S, int P, float inv_tau) {
  using Lds = BwdLds<DK, DV, M>;
  using ST = StateTiles<DK, DV, M, 4>;
  constexpr int GPW = M / NW;
  constexpr int MT = M / 16;
  constexpr size_t NE = (size_t)M * (DK + DV);
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  bf16_t* sQ = reinterpret_cast<bf16_t*>(smem + Lds::oQ);
  bf16_t* sK = reinterpret_cast<bf16_t*>(smem + Lds::oK);
  bf16_t* sV = reinterpret_cast<bf16_t*>(smem + Lds::oV);
  bf16_t* sDo = reinterpret_cast<bf16_t*>(smem + Lds::oDo);
  bf16_t* sW = reinterpret_cast<bf16_t*>(smem + Lds::oW);
  bf16_t* sX = reinterpret_cast<bf16_t*>(smem + Lds::oX);
  bf16_t* sZ = reinterpret_cast<bf16_t*>(smem + Lds::oZ);
  float* sE = reinterpret_cast<float*>(smem + Lds::oE);
  bf16_t* sS = reinterpret_cast<bf16_t*>(smem + Lds::oS);
  bf16_t* sDZ = reinterpret_cast<bf16_t*>(smem + Lds::oDZ);
  float* sDec = reinterpret_cast<float*>(smem + Lds::oDec);
  float* sCarry = reinterpret_cast<float*>(smem + Lds::oAux);  // [2][M]
  float* sWt = reinterpret_cast<float*>(smem + Lds::oWt);      // [4][M]
  float* sD = reinterpret_cast<float*>(smem + Lds::oD);
  float* sLa = reinterpret_cast<float*>(smem + Lds::oX);
  int* sFlag = reinterpret_cast<int*>(smem + Lds::oFlag);

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const bool is_state = wv >= 4;
  const int sw = wv - 4;
  const int slot0 = wv * GPW;
  const int seg = blockIdx.x % P, unit = blockIdx.x / P;
  const int nchunks = (T + C - 1) / C;
  const int c_begin = seg * S, c_end = min(c_begin + S, nchunks);
  constexpr int GS = M * G;  // gate row pitch (slot groups as in bwd_bf16_fwd)
  const int grp = unit % G;
  const size_t ub = (size_t)(unit / G) * T, wb = (size_t)unit * T;
  const bf16_t* qb = qq + ub * DK;
  const bf16_t* kb = kk + ub * DK;
  const bf16_t* vb = vv + ub * DV;
  const bf16_t* db = dOo + ub * DV;
  const bf16_t* gb = gg + ub * GS + grp * M;
  GradT<G>* dkb = dk + (ub * G + grp) * DK;
  GradT<G>* dvb = dv + (ub * G + grp) * DV;
  bf16_t* dgb = dg + ub * GS + grp * M;
  auto rows_of = [&](int ch) { return min(C, T - ch * C); };

  typedef GateRow<GPW> Row;
  Row gr, sr, zr;  // gate logits, s and dz of token row = lane, this wave's slots
  Tile<DK> pq, pk;
  Tile<DV> pv, pd;
  auto load_chunk = [&](int ch, int lane_, int tid_) {
    const int t0 = ch * C, rv = rows_of(ch);
    pq.load(qb + (size_t)t0 * DK, rv, tid_);
    pk.load(kb + (size_t)t0 * DK, rv, tid_);
    pv.load(vb + (size_t)t0 * DV, rv, tid_);
    pd.load(db + (size_t)t0 * DV, rv, tid_);
    const size_t tr = t0 + min(lane_, rv - 1);
    gr.load(gb + tr * GS + slot0);
    sr.load(s_ws + (wb + tr) * M + slot0);
    zr.load(dz_ws + (wb + tr) * M + slot0);
  };
  // stage chunk ch: tiles, factors, s*E and dz*E (zero past the end, E from
  // each token's reference point); barrier A; log alpha for an exact chunk;
  // the loads of the chunk before; returns the chunk's regime bits
  auto stage = [&](int ch, int it, int lane_, int tid_) -> int {
    const int rv = rows_of(ch);
    pq.store(sQ, Lds::LDQ, rv, tid_);
    pk.store(sK, Lds::LDQ, rv, tid_);
    pv.store(sV, Lds::LDV, rv, tid_);
    pd.store(sDo, Lds::LDV, rv, tid_);
    gr.pin();
    sr.pin();
    zr.pin();
    float E[GPW];
    const bool ok = lane_ < rv;
    const int small = chunk_factors<GPW, Lds::LDX, Lds::LDE, M>(gr, ok, inv_tau, lane_, slot0, sX, sZ, sE, sD,
                                                                 sDec, E);
    float se[GPW], ze[GPW];
#pragma unroll
    for (int s = 0; s < GPW; s++) {
      se[s] = ok ? sr.at(s) * E[s] : 0.f;
      ze[s] = ok ? zr.at(s) * E[s] : 0.f;
    }
    store_bf16_row<GPW>(sS + lane_ * Lds::LDX + slot0, se);
    store_bf16_row<GPW>(sDZ + lane_ * Lds::LDX + slot0, ze);
    const int regime = block_or(small, sFlag, it, lane_, wv);
    if (regime & kNeedExact) {
      float la[GPW];
      log_alpha_row<GPW>(gr, ok, inv_tau, la);
      store_f32_row<GPW>(sLa + lane_ * M + slot0, la);
    }
    load_chunk(max(ch - 1, c_begin), lane_, tid_);  // the chunk before (this one again at the end)
    return regime;
  };

  load_chunk(c_end - 1, lane, tid);
  if (is_state) {
    ST W;  // the adjoint of the state at the end of the current chunk
    {
      // carry from the tokens after this segment: <dW_end, W_end> per slot
      // (W_end: the next segment's start state, or the final state)
      const size_t o = ((size_t)unit * P + seg) * NE;
      W.load_w(rm + o, sw, lane);
      typename ST::MapRegs we;
      W.load_map(we, seg + 1 < P ? st + o + NE : fin + (size_t)unit * NE, sw, lane);
      float p[MT];
#pragma unroll
      for (int ct = 0; ct < MT; ct++) {
        p[ct] = 0.f;
#pragma unroll
        for (int n = 0; n < ST::NCW; n++)
#pragma unroll
          for (int i = 0; i < 4; i++) p[ct] += W.st[n][ct][i] * we[n][ct][i];
        p[ct] = group4_sum(p[ct]);
      }
      if ((lane >> 4) == 0) {
#pragma unroll
        for (int ct = 0; ct < MT; ct++) sWt[sw * M + 16 * ct + (lane & 15)] = p[ct];
      }
    }
    __syncthreads();  // the carry's partial dots
    if (sw == 0 && lane < M) sCarry[lane] = sWt[lane] + sWt[M + lane] + sWt[2 * M + lane] + sWt[3 * M + lane];
    for (int ch = c_end - 1, it = 0; ch >= c_begin; ch--, it++) {
      int lane_i = lane, tid_i = tid;
      asm volatile("" : "+v"(lane_i), "+v"(tid_i));
      const int t0 = ch * C, rv = rows_of(ch);
      W.store_copy(sW, Lds::LDW, sw, lane_i);  // the adjoint at the chunk end, for the pass waves
      const int regime = stage(ch, it, lane_i, tid_i);
      if (!(regime & kNeedExact)) {
        // the adjoint at the chunk start: Diag(E_C) dW + [Q | dO]^T [dz*E | s*E]
        if (!(regime & kNeedSub))
          W.update2(sQ, Lds::LDQ, sDo, Lds::LDV, sDZ, sS, Lds::LDX, sDec, sw, lane_i);
        else
          W.update2_sub(sQ, Lds::LDQ, sDo, Lds::LDV, sDZ, sS, Lds::LDX, sDec, sD, sw, lane_i);
      } else {
        __syncthreads();  // log alpha is in LDS
        rev_exact_state<DK, DV, M, G>(W, rv, smem, s_ws + (wb + t0) * M, dz_ws + (wb + t0) * M,
                                      dkb + (size_t)t0 * (DK * G), dvb + (size_t)t0 * (DV * G), lane_i, sw);
      }
      __syncthreads();  // B
      if (sw == 0 && lane_i < M) {  // the carry into the chunk before
        const float* carry = sCarry + (it & 1) * M;
        sCarry[((it + 1) & 1) * M + lane_i] = carry[lane_i] + sWt[lane_i] + sWt[M + lane_i] +
                                              sWt[2 * M + lane_i] + sWt[3 * M + lane_i];
      }
    }
  } else {
    __syncthreads();  // the carry's partial dots
    float pre[MT][4], sn[MT][4];
    for (int ch = c_end - 1, it = 0; ch >= c_begin; ch--, it++) {
      int lane_i = lane, tid_i = tid;
      asm volatile("" : "+v"(lane_i), "+v"(tid_i));
      const int t0 = ch * C, rv = rows_of(ch);
      const float* carry = sCarry + (it & 1) * M;
      const int regime = stage(ch, it, lane_i, tid_i);
      const bool slow = regime & kNeedExact;
      const bf16_t* hrow = h_ws + (wb + t0) * M;
      const bf16_t* grow = gb + (size_t)t0 * GS;
      GradT<G>* dkrow = dkb + (size_t)t0 * (DK * G);
      GradT<G>* dvrow = dvb + (size_t)t0 * (DV * G);
      bf16_t* dgrow = dgb + (size_t)t0 * GS;
      if (!slow) {
#define GSA_REV_PASS(JJ, SB) \
  rev_pass<DK, DV, M, JJ, G, SB>(lane_i, smem, sWt, hrow, grow, dkrow, dvrow, rv, inv_tau, pre, sn)
        if (!(regime & kNeedSub)) {
          switch (wv) {
            case 0: GSA_REV_PASS(0, false); break;
            case 1: GSA_REV_PASS(1, false); break;
            case 2: GSA_REV_PASS(2, false); break;
            default: GSA_REV_PASS(3, false); break;
          }
        } else {  // sub-chunk reference points
          switch (wv) {
            case 0: GSA_REV_PASS(0, true); break;
            case 1: GSA_REV_PASS(1, true); break;
            case 2: GSA_REV_PASS(2, true); break;
            default: GSA_REV_PASS(3, true); break;
          }
        }
#undef GSA_REV_PASS
      } else {
        __syncthreads();  // log alpha is in LDS
        rev_exact_pass<M, G>(rv, smem, Lds::oS, carry, sWt, hrow, grow, dgrow, inv_tau, lane_i, wv);
      }
      __syncthreads();  // B: every wave's gate totals are in LDS
      if (!slow) {
        switch (wv) {
          case 0: rev_pass_finish<M, 0, G>(lane_i, sWt, carry, dgrow, rv, pre, sn); break;
          case 1: rev_pass_finish<M, 1, G>(lane_i, sWt, carry, dgrow, rv, pre, sn); break;
          case 2: rev_pass_finish<M, 2, G>(lane_i, sWt, carry, dgrow, rv, pre, sn); break;
          default: rev_pass_finish<M, 3, G>(lane_i, sWt, carry, dgrow, rv, pre, sn); break;
        }
      }
    }
  }
}

// ------------------------------------------------------------ host side
// Chunks per segment: about 256 workgroups over the units (the forward's
// split), and at most kMaxSegChunks.  The gate sums inside a segment add up
// bf16-rounded per-token terms (h) and MFMA-formed di; between segments the
// carry is the exact per-slot dot of adjoint and state, so capping the
// segment bounds how many rounded terms any gate gradient sums (measured:
// 257-chunk segments, at 1024 units of 16385 tokens, reached 3.7e-2 of
// max |dg|).
constexpr int kMaxSegChunks = 8;
inline int chunks_per_segment(long long units, int nchunks) {
  if (nchunks <= 1 || units <= 0) return nchunks > 0 ? nchunks : 1;
  long long p = 256 / units;
  if (p < 1) p = 1;
  if (p > nchunks) p = nchunks;
  const int s = (int)((nchunks + p - 1) / p);
  return s < kMaxSegChunks ? s : kMaxSegChunks;
}

struct Ws {
  float *st, *dec, *fin, *rm, *rdec;
  bf16_t *s, *dz, *h;
};

inline size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace of the dense bf16 backward (bytes) and its carving: segment start
// states, the final state and reverse maps (fp32), segment decays, and s, dz,
// h per token (bf16).
inline size_t ws_bytes(size_t U, int T, int dk, int dv, int m, Ws* w = nullptr, void* base = nullptr) {
  const int nchunks = (T + C - 1) / C;
  const int S = chunks_per_segment((long long)U, nchunks);
  const size_t P = (size_t)((nchunks + S - 1) / S);
  const size_t NE = (size_t)m * (dk + dv);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += a256(bytes);
    return o;
  };
  const size_t o_st = take(U * P * NE * 4), o_dec = take(U * P * m * 4), o_fin = take(U * NE * 4),
               o_rm = take(U * P * NE * 4),
               o_rdec = take(U * P * m * 4), o_s = take(U * T * (size_t)m * 2),
               o_dz = take(U * T * (size_t)m * 2), o_h = take(U * T * (size_t)m * 2);
  if (w) {
    char* b = (char*)base;
    w->st = (float*)(b + o_st);
    w->dec = (float*)(b + o_dec);
    w->fin = (float*)(b + o_fin);
    w->rm = (float*)(b + o_rm);
    w->rdec = (float*)(b + o_rdec);
    w->s = (bf16_t*)(b + o_s);
    w->dz = (bf16_t*)(b + o_dz);
    w->h = (bf16_t*)(b + o_h);
  }
  return off;
}

// Two slot groups (m = 2M): besides the groups' own workspace (2U units), the
// groups' softmax statistics per token ([rows][2][2] fp32), the merged
// log-sum-exp and delta per token, and the groups' partial dq, dk, dv
// ([rows][2][d] fp32).
struct GroupWs {
  float *dq, *dk, *dv;
  float *stats, *lse, *delta;
};

inline size_t ws_bytes_groups(size_t U, int T, int dk, int dv, int m, Ws* w = nullptr, GroupWs* gw = nullptr,
                              void* base = nullptr) {
  size_t off = a256(ws_bytes(2 * U, T, dk, dv, m, w, base));
  const size_t rows = U * (size_t)T;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += a256(bytes);
    return o;
  };
  const size_t o_stats = take(rows * 4 * 4), o_lse = take(rows * 4), o_delta = take(rows * 4),
               o_dq = take(rows * 2 * dk * 4), o_dk = take(rows * 2 * dk * 4), o_dv = take(rows * 2 * dv * 4);
  if (gw) {
    char* b = (char*)base;
    gw->stats = (float*)(b + o_stats);
    gw->lse = (float*)(b + o_lse);
    gw->delta = (float*)(b + o_delta);
    gw->dq = (float*)(b + o_dq);
    gw->dk = (float*)(b + o_dk);
    gw->dv = (float*)(b + o_dv);
  }
  return off;
}

// The softmax over all 2M slots from the two groups' own statistics per token
// (l_h = log-sum-exp over group h, A_h = sum over group h of s ds under its own
// softmax; stats [rows][2][2]): lse = log(e^{l_0} + e^{l_1}) and delta =
// w_0 A_0 + w_1 A_1 with w_h = e^{l_h - lse}, the sum of s ds over all the
// slots.  One thread per row.
__global__ void __launch_bounds__(256)
bwd_bf16_group_stats(const float* __restrict__ stats, float* __restrict__ lse, float* __restrict__ delta,
                     size_t rows) {
  const size_t row = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (row >= rows) return;
  const float4 x = *reinterpret_cast<const float4*>(stats + 4 * row);
  const float mx = fmaxf(x.x, x.z);
  const float e0 = __expf(x.x - mx), e1 = __expf(x.z - mx);
  const float inv = 1.f / (e0 + e1);
  lse[row] = mx + __logf(e0 + e1);
  delta[row] = (e0 * x.y + e1 * x.w) * inv;
}

// dx = x_0 + x_1 over the two slot groups' partial gradients: blockIdx.y
// picks dq, dk or dv; p [rows][2][D] fp32 -> o [rows][D] bf16.  Thread = 4
// columns of one row.
template <int D>
__global__ void __launch_bounds__(256)
bwd_bf16_group_sum(const float* __restrict__ p0, bf16_t* __restrict__ o0, const float* __restrict__ p1,
                   bf16_t* __restrict__ o1, const float* __restrict__ p2, bf16_t* __restrict__ o2, size_t rows) {
  constexpr int TPR = D / 4;
  const size_t gid = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t row = gid / TPR;
  const int c = (int)(gid % TPR) * 4;
  if (row >= rows) return;
  const float* p = blockIdx.y == 0 ? p0 : blockIdx.y == 1 ? p1 : p2;
  bf16_t* o = blockIdx.y == 0 ? o0 : blockIdx.y == 1 ? o1 : o2;
  const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + (2 * row) * D + c));
  const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + (2 * row + 1) * D + c));
  st_grad4(o + row * D + c, a + b);
}

// G = 1: the dense batch.  G = 2: m = 2M slots as two groups (unit 2u + h);
// for the softmax read a statistics pass of the forward sweep and a merge
// give the log-sum-exp over all slots and delta (the sum of s ds over all
// slots) per token, which both groups' backward passes take, and the groups'
// partial dq, dk, dv are summed last.
template <int DK, int DV, int M, int ACT, int G>
int launch(const GsaBwdLaunch& a) {
  using Lds = BwdLds<DK, DV, M>;
  const int U = a.B * a.H * G, T = a.T;  // (group) units
  const int nchunks = (T + C - 1) / C;
  const int S = chunks_per_segment(U, nchunks);
  const int P = (nchunks + S - 1) / S;
  Ws w;
  GroupWs gw{};
  if constexpr (G > 1)
    ws_bytes_groups((size_t)a.B * a.H, T, DK, DV, M, &w, &gw, a.ws);
  else
    ws_bytes((size_t)U, T, DK, DV, M, &w, a.ws);
  const float inv_tau = 1.0f / a.tau;
  static const bool lds_set = [] {
    (void)hipFuncSetAttribute((const void*)bwd_bf16_fwd<DK, DV, M, ACT, G, false>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, Lds::total);
    if constexpr (G > 1 && ACT == kActSoftmax)
      (void)hipFuncSetAttribute((const void*)bwd_bf16_fwd<DK, DV, M, ACT, G, true>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, Lds::total);
    (void)hipFuncSetAttribute((const void*)bwd_bf16_rev<DK, DV, M, G>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              Lds::total);
    return true;
  }();
  (void)lds_set;
  if (a.saved_states)  // the training forward's start states (same split), read only
    w.st = const_cast<float*>(a.saved_states);
  else if (gsa_bf16_segment_states(DK, DV, M, G, a.k, a.v, a.g, a.k0, a.v0, w.st, w.dec, U, T, S, P, a.tau,
                                   a.stream) != 0)
    return -1;
  const bf16_t *q = (const bf16_t*)a.q, *k = (const bf16_t*)a.k, *v = (const bf16_t*)a.v, *g = (const bf16_t*)a.g,
               *dO = (const bf16_t*)a.d_o;
  if constexpr (G > 1 && ACT == kActSoftmax) {
    hipLaunchKernelGGL((bwd_bf16_fwd<DK, DV, M, ACT, G, true>), dim3(P * U), dim3(NT), Lds::total,
                       (hipStream_t)a.stream, q, k, v, g, dO, (const float*)w.st, w.fin, w.rm, w.rdec,
                       (GradT<G>*)nullptr, w.s, w.dz, w.h, T, S, P, inv_tau, (const float*)nullptr,
                       (const float*)nullptr, gw.stats);
    const size_t rows = (size_t)a.B * a.H * T;
    hipLaunchKernelGGL(bwd_bf16_group_stats, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0,
                       (hipStream_t)a.stream, (const float*)gw.stats, gw.lse, gw.delta, rows);
  }
  GradT<G>* dq;
  GradT<G>* dk;
  GradT<G>* dv;
  if constexpr (G > 1) {
    dq = gw.dq;
    dk = gw.dk;
    dv = gw.dv;
  } else {
    dq = (bf16_t*)a.dq;
    dk = (bf16_t*)a.dk;
    dv = (bf16_t*)a.dv;
  }
  launch_timed(bwd_bf16_fwd<DK, DV, M, ACT, G, false>, dim3(P * U), dim3(NT), Lds::total, a.stream, a.events, 0,
               1, q, k, v, g, dO, (const float*)w.st, w.fin, w.rm, w.rdec, dq, w.s, w.dz, w.h, T, S, P, inv_tau,
               (const float*)gw.lse, (const float*)gw.delta, (float*)nullptr);
  const long long ne = (long long)U * M * (DK + DV) / 4;
  hipLaunchKernelGGL((bwd_bf16_rscan<DK, DV, M>), dim3((unsigned)((ne + 255) / 256)), dim3(256), 0,
                     (hipStream_t)a.stream, w.rm, (const float*)w.rdec, a.dkf, a.dvf, a.dk0, a.dv0, U, P);
  launch_timed(bwd_bf16_rev<DK, DV, M, G>, dim3(P * U), dim3(NT), Lds::total, a.stream, a.events, 2, 3, q, k, v,
               g, dO, (const float*)w.st, (const float*)w.fin, (const float*)w.rm, (const bf16_t*)w.s,
               (const bf16_t*)w.dz,
               (const bf16_t*)w.h, dk, dv, (bf16_t*)a.dg, T, S, P, inv_tau);
  if constexpr (G > 1) {
    static_assert(DK == DV, "one row width for the three sums");
    const size_t rows = (size_t)a.B * a.H * T;
    const size_t threads = rows * (DK / 4);
    hipLaunchKernelGGL((bwd_bf16_group_sum<DK>), dim3((unsigned)((threads + 255) / 256), 3), dim3(256), 0,
                       (hipStream_t)a.stream, (const float*)gw.dq, (bf16_t*)a.dq, (const float*)gw.dk,
                       (bf16_t*)a.dk, (const float*)gw.dv, (bf16_t*)a.dv, rows);
  }
  return 0;
}

template <int DK, int DV, int M, int G>
int launch_act(const GsaBwdLaunch& a) {
  switch (a.act) {
    case kActSoftmax: return launch<DK, DV, M, kActSoftmax, G>(a);
    case kActIdentity: return launch<DK, DV, M, kActIdentity, G>(a);
    case kActSwish: return launch<DK, DV, M, kActSwish, G>(a);
    case kActRelu: return launch<DK, DV, M, kActRelu, G>(a);
    case kActRelu2: return launch<DK, DV, M, kActRelu2, G>(a);
    default: return -1;
  }
}

}  // namespace bfb

int gsa_bwd_chunks_per_segment(long long units, int nchunks) { return bfb::chunks_per_segment(units, nchunks); }

// The dense bf16 backward on the matrix cores: returns the workspace bytes
// (query) or launches (0); -1 if (dk, dv, m) is not compiled for it.
long long gsa_bwd_bf16_dispatch(int dk, int dv, int m, const GsaBwdLaunch* a, bool query, size_t units, int T) {
#define BWD_BF16_CASE(DKC, DVC, MC)                                                        \
  if (dk == DKC && dv == DVC && m == MC)                                                   \
    return query ? (long long)bfb::ws_bytes(units, T, DKC, DVC, MC) : bfb::launch_act<DKC, DVC, MC, 1>(*a);
  // m = 2 * 64 as two slot groups (slot_groups(1, 128) == 2)
#define BWD_BF16_GROUPS_CASE(DKC, DVC, MC)                                                        \
  if (dk == DKC && dv == DVC && m == 2 * MC)                                                      \
    return query ? (long long)bfb::ws_bytes_groups(units, T, DKC, DVC, MC) : bfb::launch_act<DKC, DVC, MC, 2>(*a);
  BWD_BF16_GROUPS_CASE(128, 128, 64)
  BWD_BF16_GROUPS_CASE(64, 64, 64)
  BWD_BF16_CASE(128, 128, 64)
  BWD_BF16_CASE(128, 128, 32)
  BWD_BF16_CASE(64, 64, 64)
  BWD_BF16_CASE(64, 64, 32)
#undef BWD_BF16_CASE
#undef BWD_BF16_GROUPS_CASE
  return -1;
}

}  // namespace gsa
