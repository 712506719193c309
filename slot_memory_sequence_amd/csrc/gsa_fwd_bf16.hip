// Chunkwise GSA forward on gfx950, bf16 inputs, fp32 state and accumulation.
//
// Method: "Gated Slot Attention for Efficient Linear-Time Sequence Modeling"
// (arXiv 2409.07146), Sec. 3.2 (two gated passes over m slots linked by a
// softmax over the slots), Sec. 3.3 (alpha = sigmoid(g)^(1/tau)), App. A.1
// (chunk form: a read of the chunk-start state plus a causal intra-chunk term)
// and App. B (the two passes as GLA calls; chunk-local cumulative decay).
//
// Per chunk of C = 64 tokens, with E_j = prod_{i<=j} alpha_i and
// S_r = prod_{i>r} alpha_i per slot (chunk-local), X = (1-alpha) / E and
// Z = (1-alpha) * S, and the state W = [Kt | Vt] in R^{m x (dk+dv)}:
//   pass 1   o'^T = E^T * ( Wk Q^T + X^T mask(K Q^T) )          [m x C]
//   softmax  s    = softmax over slots of o'   (columns of o'^T)
//   pass 2   o^T  = Wv^T (s*E)^T + V^T mask( X (s*E)^T )          [dv x C]
//   carry    W^T <- W^T Diag(E_C) + [K|V]^T Z                     [(dk+dv) x m]
// Everything is computed transposed so that (a) the masked score blocks leave
// the matrix cores in exactly the register layout the next contraction takes
// as an operand (the contraction index is permuted consistently on both
// operands), (b) the slot softmax of a token is a reduction inside one wave,
// and (c) the output rows are written as 8-byte vectors.
//
// Wave roles inside the 512-thread workgroup:
//   waves 0..3 ("pass"): token rows 16J..16J+15 of the chunk (J = wave), both
//              passes and the softmax, all in registers;
//   waves 4..7 ("state"): the fp32 state W^T in MFMA accumulators, a quarter of
//              its columns each, and the bf16 copy of W that the pass waves read.
// Two workgroup barriers per chunk.
//
// Launches (no inter-workgroup waiting): state maps of the segments
// (gsa_bf16_state), a per-unit fp32 scan over the segments (gsa_bf16_scan) and
// the outputs (gsa_bf16_out).  With at most kMaxFoldedMaps maps before the last
// segment there is no scan launch: each output workgroup folds the maps before
// its segment into its start state (a dependent launch costs more than a few
// such reads); a training forward that keeps its start states for the
// backward always launches the scan (into the caller's buffer).  A chunk
// whose decay product falls below 2^-90 in some slot is run with 16-token
// sub-chunk reference points (App. A.1, secondary chunking: the same
// contractions, with the intra-chunk terms carried between the reference
// points by the sub-chunk decays), and one in which a 16-token sub-chunk decays
// below 2^-90 as the exact token recurrence (no division by a decay product).
// 128 slots run
// as two groups of 64, each its own unit of these kernels (SlotGroups), and
// gsa_bf16_merge combines the groups' outputs by their log-sum-exps.
#include <algorithm>
#include <type_traits>

#include "bf16_common.hpp"
#include "bf16_state.hpp"
#include "common.hpp"
#include "internal.hpp"
#include "launch.hpp"

namespace gsa {
namespace bfk {

// --------------------------------------------------------------- LDS plans
template <int DK, int DV, int M>
struct OutLds {
  static constexpr int PAD = 8;
  static constexpr int LDQ = DK + PAD, LDV = DV + PAD, LDW = DK + DV + PAD, LDX = M + PAD;
  static constexpr int LDE = M + 4;
  static constexpr int oQ = 0;
  static constexpr int oK = oQ + C * LDQ * 2;
  static constexpr int oV = oK + C * LDQ * 2;
  static constexpr int oR = oV + C * LDV * 2;          // region used differently by the two paths
  // fast path: bf16 copy of W, then two sets of chunk factors (this chunk's
  // and the next one's, computed while this chunk is processed)
  static constexpr int oW = oR;                        // bf16 W [M][DK+DV]
  static constexpr int oF = oW + M * LDW * 2;
  static constexpr int fX = 0;                         // X [C][M] bf16
  static constexpr int fZ = fX + C * LDX * 2;          // Z [C][M] bf16
  static constexpr int fE = fZ + C * LDX * 2;          // E [C][M] fp32
  static constexpr int fD = fE + C * LDE * 4;          // decays between reference points [4][M] fp32
  static constexpr int szF = fD + 4 * M * 4;           // one factor set
  static constexpr int szFast = oF + 2 * szF - oR;
  // exact-recurrence path
  static constexpr int oWf = oR;                       // fp32 W [M][DK+DV]
  static constexpr int oLa = oWf + M * (DK + DV) * 4;  // log alpha [C][M] fp32
  static constexpr int oZs = oLa + C * M * 4;          // slot scores [M] fp32
  static constexpr int oOp = oZs + M * 4;              // output partials [NW][DV] fp32
  static constexpr int szSlow = oOp + NW * DV * 4 - oR;
  static constexpr int oDec = oR + (szFast > szSlow ? szFast : szSlow);  // 2 x [M] fp32
  static constexpr int oFlag = oDec + 2 * M * 4;                         // 2 x NW ints
  static constexpr int total = oFlag + 2 * NW * 4;
  static_assert(oK % 16 == 0 && oV % 16 == 0 && oW % 16 == 0 && oF % 16 == 0 && szF % 16 == 0 &&
                    fZ % 16 == 0 && fE % 16 == 0 && fD % 16 == 0 && oLa % 16 == 0 && oOp % 16 == 0 && oDec % 16 == 0,
                "LDS tiles must stay 16-byte aligned");
};

template <int DK, int DV, int M>
struct StateLds {  // two buffers of everything a chunk needs (software pipeline)
  static constexpr int PAD = 8;
  static constexpr int LDQ = DK + PAD, LDV = DV + PAD, LDX = M + PAD;
  static constexpr int oK = 0;
  static constexpr int oV = oK + C * LDQ * 2;
  static constexpr int oZ = oV + C * LDV * 2;
  static constexpr int oDec = oZ + C * LDX * 2;
  static constexpr int szBuf = oDec + M * 4;
  static constexpr int total = 2 * szBuf;
  static_assert(oV % 16 == 0 && oZ % 16 == 0 && oDec % 16 == 0 && szBuf % 16 == 0, "alignment");
};

// -------------------------------------------------------- pass-wave chunk
// Token rows 16J..16J+15 of the chunk: pass 1, the slot read non-linearity
// (ACT: the softmax, or an element-wise ablation function), pass 2 and the
// output rows.  Reads sQ, sK, sV, sX, sE and the bf16 state copy sW.  J is a
// template parameter so that every loop is static and independent
// accumulators can be interleaved.  G > 1 (slot groups): output rows have the
// pitch G * DV, and the softmax's log-sum-exp of token j goes to lrow[j * G].
// SUB: the sub-chunk form of the reads (chunk_factors): the intra-chunk sums
// run per 16-token sub-chunk R <= J, and a term of sub-chunk R is carried to
// this wave's reference point by the decays sD[R] ... sD[J-1] between them --
// in pass 1 by scaling the running slot scores before each sub-chunk is added
// (the state read counts as the term before sub-chunk 0), in pass 2 by
// scaling the weights s*E before the scores of each sub-chunk are formed.
template <int DK, int DV, int M, int J, int ACT, int G, bool SUB>
__device__ __forceinline__ void pass_chunk(int lane, const bf16_t* sQ, const bf16_t* sK,
                                           const bf16_t* sV, const bf16_t* sW, const bf16_t* sX,
                                           const float* sE, const float* sD, bf16_t* __restrict__ orow,
                                           float* __restrict__ lrow, int rv) {
  using Lds = OutLds<DK, DV, M>;
  constexpr int MT = M / 16, KQ = DK / 32, NP = M / 32, NVT = DV / 16;
  constexpr int NR = J + 1;         // score row tiles r <= j
  constexpr int NPR = J / 2 + 1;    // r-tile pairs
  const int L = lane & 15, g = lane >> 4;
  const int j = 16 * J + L;  // this lane's token column

  // Q^T operand: B[d][j] = Q[j][d]
  bf16x8 qf[KQ];
#pragma unroll
  for (int s = 0; s < KQ; s++) qf[s] = ld_row(sQ, Lds::LDQ, 16 * J, 32 * s, lane);

  // A^T[r][j] = k_r . q_j for row tiles R <= J, causal mask on the diagonal tile
  f32x4 at[4];
#pragma unroll
  for (int R = 0; R < 4; R++) at[R] = zero4();
#pragma unroll
  for (int s = 0; s < KQ; s++)
#pragma unroll
    for (int R = 0; R < NR; R++) at[R] = mma(ld_row(sK, Lds::LDQ, 16 * R, 32 * s, lane), qf[s], at[R]);
#pragma unroll
  for (int i = 0; i < 4; i++)
    if (4 * g + i > L) at[J][i] = 0.f;

  // pass 1: o'^T[c][j] = E[j][c] (Wk[c].q_j + sum_r X[r][c] A^T[r][j])
  f32x4 op[MT];
#pragma unroll
  for (int ct = 0; ct < MT; ct++) op[ct] = zero4();
#pragma unroll
  for (int s = 0; s < KQ; s++)
#pragma unroll
    for (int ct = 0; ct < MT; ct++) op[ct] = mma(ld_row(sW, Lds::LDW, 16 * ct, 32 * s, lane), qf[s], op[ct]);
  if constexpr (!SUB) {
    bf16x8 af[2];
    af[0] = pack8(at[0], at[1]);
    af[1] = pack8(at[2], at[3]);
#pragma unroll
    for (int pr = 0; pr < NPR; pr++)
#pragma unroll
      for (int ct = 0; ct < MT; ct++)
        op[ct] = mma(ld_col(sX, Lds::LDX, 16 * ct, 32 * pr + 4 * g, 32 * pr + 16 + 4 * g, lane), af[pr], op[ct]);
  } else {
#pragma unroll
    for (int R = 0; R < NR; R++) {
      if (R > 0) {
#pragma unroll
        for (int ct = 0; ct < MT; ct++) {
          const float4 dd = *reinterpret_cast<const float4*>(sD + (R - 1) * M + 16 * ct + 4 * g);
          op[ct][0] *= dd.x;
          op[ct][1] *= dd.y;
          op[ct][2] *= dd.z;
          op[ct][3] *= dd.w;
        }
      }
      const bf16x4v ar = pack4(at[R]);
#pragma unroll
      for (int ct = 0; ct < MT; ct++) op[ct] = mma16(ld_col4(sX, Lds::LDX, 16 * ct, 16 * R + 4 * g, lane), ar, op[ct]);
    }
  }
#pragma unroll
  for (int ct = 0; ct < MT; ct++) {
    const float4 e = *reinterpret_cast<const float4*>(sE + j * Lds::LDE + 16 * ct + 4 * g);
    op[ct][0] *= e.x;
    op[ct][1] *= e.y;
    op[ct][2] *= e.z;
    op[ct][3] *= e.w;
  }

  float inv = 1.f;
  if constexpr (ACT == kActSoftmax) {
    // slot softmax of token j: over (ct, i) in-lane and the four lane groups
    float mx = op[0][0];
#pragma unroll
    for (int ct = 0; ct < MT; ct++)
#pragma unroll
      for (int i = 0; i < 4; i++) mx = fmaxf(mx, op[ct][i]);
    mx = group4_max(mx);
    float sm = 0.f;
#pragma unroll
    for (int ct = 0; ct < MT; ct++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        op[ct][i] = __builtin_amdgcn_exp2f((op[ct][i] - mx) * 1.4426950408889634f);
        sm += op[ct][i];
      }
    sm = group4_sum(sm);
    inv = 1.f / sm;
    if constexpr (G > 1) {
      if (g == 0 && j < rv) lrow[(size_t)j * G] = mx + __logf(sm);
    }
  } else {
    // element-wise replacement of the softmax (Table 2 ablations)
#pragma unroll
    for (int ct = 0; ct < MT; ct++)
#pragma unroll
      for (int i = 0; i < 4; i++) op[ct][i] = slot_act<ACT>(op[ct][i]);
  }
  // (s*E)^T as B operands over slot pairs (permuted slot index), and the
  // pass 2 scores A2^T[r][j] = sum_c X[r][c] (s*E)[j][c], r tiles R <= J
  bf16x8 sb[NP];
  f32x4 a2[4];
#pragma unroll
  for (int R = 0; R < 4; R++) a2[R] = zero4();
  if constexpr (!SUB) {
#pragma unroll
    for (int p = 0; p < NP; p++) {
      const float4 ea = *reinterpret_cast<const float4*>(sE + j * Lds::LDE + 32 * p + 4 * g);
      const float4 eb = *reinterpret_cast<const float4*>(sE + j * Lds::LDE + 32 * p + 16 + 4 * g);
      const f32x4 a = {op[2 * p][0] * inv * ea.x, op[2 * p][1] * inv * ea.y, op[2 * p][2] * inv * ea.z,
                       op[2 * p][3] * inv * ea.w};
      const f32x4 b = {op[2 * p + 1][0] * inv * eb.x, op[2 * p + 1][1] * inv * eb.y,
                       op[2 * p + 1][2] * inv * eb.z, op[2 * p + 1][3] * inv * eb.w};
      sb[p] = pack8(a, b);
    }
#pragma unroll
    for (int p = 0; p < NP; p++)
#pragma unroll
      for (int R = 0; R < NR; R++)
        a2[R] = mma(ld_row2(sX, Lds::LDX, 16 * R, 32 * p + 4 * g, 32 * p + 16 + 4 * g, lane), sb[p], a2[R]);
  } else {
    // weights at this wave's reference point, then carried back one sub-chunk
    // at a time: the last set (R = 0) is s*E from the chunk start, which the
    // state read below takes as well
#pragma unroll
    for (int ct = 0; ct < MT; ct++) {
      const float4 e = *reinterpret_cast<const float4*>(sE + j * Lds::LDE + 16 * ct + 4 * g);
      op[ct][0] *= inv * e.x;
      op[ct][1] *= inv * e.y;
      op[ct][2] *= inv * e.z;
      op[ct][3] *= inv * e.w;
    }
#pragma unroll
    for (int R = NR - 1; R >= 0; R--) {
      if (R < J) {
#pragma unroll
        for (int ct = 0; ct < MT; ct++) {
          const float4 dd = *reinterpret_cast<const float4*>(sD + R * M + 16 * ct + 4 * g);
          op[ct][0] *= dd.x;
          op[ct][1] *= dd.y;
          op[ct][2] *= dd.z;
          op[ct][3] *= dd.w;
        }
      }
#pragma unroll
      for (int p = 0; p < NP; p++) sb[p] = pack8(op[2 * p], op[2 * p + 1]);
#pragma unroll
      for (int p = 0; p < NP; p++)
        a2[R] = mma(ld_row2(sX, Lds::LDX, 16 * R, 32 * p + 4 * g, 32 * p + 16 + 4 * g, lane), sb[p], a2[R]);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; i++)
    if (4 * g + i > L) a2[J][i] = 0.f;
  bf16x8 a2f[2];
  a2f[0] = pack8(a2[0], a2[1]);
  a2f[1] = pack8(a2[2], a2[3]);

  // o^T[n][j] = sum_c Wv[c][n] (s*E)[j][c] + sum_r V[r][n] A2^T[r][j], in
  // groups of four column tiles
  const bool store = j < rv;
  constexpr int NG = NVT < 4 ? NVT : 4;
#pragma unroll
  for (int n0 = 0; n0 < NVT; n0 += NG) {
    f32x4 acc[NG];
#pragma unroll
    for (int u = 0; u < NG; u++) acc[u] = zero4();
#pragma unroll
    for (int p = 0; p < NP; p++)
#pragma unroll
      for (int u = 0; u < NG; u++)
        acc[u] = mma(ld_col(sW + DK, Lds::LDW, 16 * (n0 + u), 32 * p + 4 * g, 32 * p + 16 + 4 * g, lane),
                     sb[p], acc[u]);
#pragma unroll
    for (int pr = 0; pr < NPR; pr++)
#pragma unroll
      for (int u = 0; u < NG; u++)
        acc[u] = mma(ld_col(sV, Lds::LDV, 16 * (n0 + u), 32 * pr + 4 * g, 32 * pr + 16 + 4 * g, lane),
                     a2f[pr], acc[u]);
    if (store) {
#pragma unroll
      for (int u = 0; u < NG; u++)
        // streaming store: the outputs are not read again by this operation
        __builtin_nontemporal_store(__builtin_bit_cast(u32x2, pack4(acc[u])),
                                    reinterpret_cast<u32x2*>(orow + (size_t)j * (DV * G) + 16 * (n0 + u) + 4 * g));
    }
  }
}

// ------------------------------------------------ exact chunk recurrence
// Runs one chunk token by token: Kt, Vt <- Diag(alpha) (.) + (1-alpha)[k|v]^T,
// s = softmax over slots of Kt q (or the element-wise ACT), o = Vt^T s
// (Sec. 3.2 recurrent form).  Used
// for chunks in which some slot decays too fast even for the sub-chunk form.
// The state waves' accumulators W are written to LDS, advanced there by all
// threads, and read back.  Contains workgroup barriers: all threads call it.
// G as in pass_chunk.
template <int DK, int DV, int M, int ACT, int G>
__device__ __forceinline__ void exact_chunk(StateTiles<DK, DV, M, 4>& W, int rv, unsigned char* smem,
                                            const bf16_t* sQ, const bf16_t* sK, const bf16_t* sV,
                                            bf16_t* __restrict__ orow, float* __restrict__ lrow, int tid) {
  using Lds = OutLds<DK, DV, M>;
  constexpr int TPS = NT / M;            // threads per slot
  constexpr int KPT = DK / TPS, VPT = DV / TPS;
  constexpr int SPW = 64 / TPS;          // slots per wave
  static_assert(NT % M == 0 && TPS <= 64 && KPT >= 1 && VPT >= 1, "exact-path thread map");
  float* sWf = reinterpret_cast<float*>(smem + Lds::oWf);
  float* sLa = reinterpret_cast<float*>(smem + Lds::oLa);
  float* sZs = reinterpret_cast<float*>(smem + Lds::oZs);
  float* sOp = reinterpret_cast<float*>(smem + Lds::oOp);
  const int lane = tid & 63, wv = tid >> 6;
  const bool is_state = wv >= 4;
  const int sw = wv - 4;

  // the state to LDS (the region held the fast path's factors and the bf16
  // state copy, all of whose readers passed the last barrier); the caller has
  // written this chunk's log alpha to sLa
  if (is_state) W.store_w(sWf, sw, lane);
  __syncthreads();
  const int c = tid / TPS, p = tid % TPS;
  float wk[KPT], wvv[VPT];
#pragma unroll
  for (int i = 0; i < KPT; i++) wk[i] = sWf[c * (DK + DV) + p * KPT + i];
#pragma unroll
  for (int i = 0; i < VPT; i++) wvv[i] = sWf[c * (DK + DV) + DK + p * VPT + i];

  for (int jt = 0; jt < rv; jt++) {
    const float la = sLa[jt * M + c];
    const float a = __expf(la), w = -expm1f(la);
    float z = 0.f;
#pragma unroll
    for (int i = 0; i < KPT; i++) {
      wk[i] = a * wk[i] + w * bf2f(sK[jt * Lds::LDQ + p * KPT + i]);
      z += wk[i] * bf2f(sQ[jt * Lds::LDQ + p * KPT + i]);
    }
#pragma unroll
    for (int off = 1; off < TPS; off <<= 1) z += __shfl_xor(z, off, 64);
    if (p == 0) sZs[c] = z;
#pragma unroll
    for (int i = 0; i < VPT; i++) wvv[i] = a * wvv[i] + w * bf2f(sV[jt * Lds::LDV + p * VPT + i]);
    __syncthreads();
    float sc;
    if constexpr (ACT == kActSoftmax) {
      // slot softmax, computed by every wave; lane l < M holds slot l
      const float zl = lane < M ? sZs[lane] : -INFINITY;
      float mx = zl;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
      const float el = lane < M ? __expf(zl - mx) : 0.f;
      const float sm = sum64(el);
      sc = __shfl(el, c, 64) / sm;
      if constexpr (G > 1) {
        if (tid == 0) lrow[(size_t)jt * G] = mx + __logf(sm);
      }
    } else {
      sc = slot_act<ACT>(sZs[c]);
    }
    // o partials: reduce over the wave's slots (lanes with equal p), then over waves
    float op[VPT];
#pragma unroll
    for (int i = 0; i < VPT; i++) {
      float x = wvv[i] * sc;
#pragma unroll
      for (int off = TPS; off < 64; off <<= 1) x += __shfl_xor(x, off, 64);
      op[i] = x;
    }
    if (lane < TPS) {
#pragma unroll
      for (int i = 0; i < VPT; i++) sOp[wv * DV + p * VPT + i] = op[i];
    }
    __syncthreads();
    if (tid < DV) {
      float o = 0.f;
#pragma unroll
      for (int w8 = 0; w8 < NW; w8++) o += sOp[w8 * DV + tid];
      orow[(size_t)jt * (DV * G) + tid] = f2bf(o);
    }
  }
  (void)SPW;
  // state back to the accumulators
#pragma unroll
  for (int i = 0; i < KPT; i++) sWf[c * (DK + DV) + p * KPT + i] = wk[i];
#pragma unroll
  for (int i = 0; i < VPT; i++) sWf[c * (DK + DV) + DK + p * VPT + i] = wvv[i];
  __syncthreads();
  if (is_state) W.load_w(sWf, sw, lane);
  __syncthreads();  // the region is reused by the next factor set
}

// ------------------------------------------------ phase A: segment maps
// grid (P-1, units).  Map of segment seg from a zero start:
// D = sum over its tokens of Diag(prod_{i>r} alpha_i)(1-alpha_r)[k_r|v_r]^T and
// the segment decay product.  All eight waves carry state columns.  A segment
// past the end of its sequence (variable-length batches) writes the identity
// map (D = 0, decay 1).
template <int DK, int DV, int M, class Seq>
__global__ void __launch_bounds__(NT, 1)
gsa_bf16_state(const bf16_t* __restrict__ kk, const bf16_t* __restrict__ vv,
               const bf16_t* __restrict__ gg, float* __restrict__ ws_state,
               float* __restrict__ ws_dec, Seq seq, int S, int P, float inv_tau) {
  using Lds = StateLds<DK, DV, M>;
  constexpr int SPT = M / NW;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  auto bK = [&](int b) { return reinterpret_cast<bf16_t*>(smem + b * Lds::szBuf + Lds::oK); };
  auto bV = [&](int b) { return reinterpret_cast<bf16_t*>(smem + b * Lds::szBuf + Lds::oV); };
  auto bZ = [&](int b) { return reinterpret_cast<bf16_t*>(smem + b * Lds::szBuf + Lds::oZ); };
  auto bDec = [&](int b) { return reinterpret_cast<float*>(smem + b * Lds::szBuf + Lds::oDec); };

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int seg = blockIdx.x, unit = seq.unit_of(blockIdx.y);
  const Span sp = seq.span(unit);
  const int T_len = sp.len;
  const int nchunks = (T_len + C - 1) / C;
  const int c_begin = seg * S, c_end = min(c_begin + S, nchunks);
  const bf16_t* kb = kk + sp.base * DK;
  const bf16_t* vb = vv + sp.base * DV;
  const bf16_t* gb = gg + gate_base<Seq, M>(sp, unit) + wv * SPT;
  constexpr int GS = M * Seq::kGroups;  // gate row pitch

  StateTiles<DK, DV, M, NW> W;
  W.zero();
  float segdec[SPT];
#pragma unroll
  for (int s = 0; s < SPT; s++) segdec[s] = 1.f;

  // stage chunk ch into buffer b: tiles from registers, gates from the logits
  Tile<DK> pk;
  Tile<DV> pv;
  GateRow<SPT> pg;
  auto load_chunk = [&](int ch, int tid_, int lane_) {
    const int t0 = ch * C, rv = min(C, T_len - t0);
    pk.load(kb + (size_t)t0 * DK, rv, tid_);
    pv.load(vb + (size_t)t0 * DV, rv, tid_);
    pg.load(gb + (size_t)(t0 + min(lane_, rv - 1)) * GS);
  };
  auto stage_chunk = [&](int ch, int b, bool count, int tid_, int lane_) {
    const int rv = min(C, T_len - ch * C);
    pk.store(bK(b), Lds::LDQ, rv, tid_);
    pv.store(bV(b), Lds::LDV, rv, tid_);
    SuffixGates<SPT> gt;
    gt.compute(pg, lane_ < rv, inv_tau);
#pragma unroll
    for (int s = 0; s < SPT; s++) {
      segdec[s] *= count ? gt.dec[s] : 1.f;
      if (lane_ == 0) bDec(b)[wv * SPT + s] = gt.dec[s];
    }
    store_bf16_row<SPT>(bZ(b) + lane_ * Lds::LDX + wv * SPT, gt.Z);
  };

  if (Seq::kVar && c_begin >= c_end) {
    // no tokens: the identity map (W and segdec as initialised)
  } else {
  load_chunk(c_begin, tid, lane);
  stage_chunk(c_begin, 0, true, tid, lane);
  load_chunk(min(c_begin + 1, c_end - 1), tid, lane);
  __syncthreads();
  int b = 0;
  for (int ch = c_begin; ch < c_end; ch++) {
    int lane_i = lane, tid_i = tid;  // re-derived per chunk (see the output kernel)
    asm volatile("" : "+v"(lane_i), "+v"(tid_i));
    // next chunk into the other buffer (the last chunk's again at the end,
    // into a buffer nobody reads), the one after into registers, this chunk's
    // state update: all independent until the barrier
    const int cn = min(ch + 1, c_end - 1);
    stage_chunk(cn, b ^ 1, ch + 1 < c_end, tid_i, lane_i);
    load_chunk(min(ch + 2, c_end - 1), tid_i, lane_i);
    W.carry(bK(b), Lds::LDQ, bV(b), Lds::LDV, bZ(b), Lds::LDX, bDec(b), wv, lane_i);
    __syncthreads();
    b ^= 1;
  }
  }
  W.store_w_nt(ws_state + ((size_t)unit * P + seg) * M * (DK + DV), wv, lane);
  if (lane == 0) {
#pragma unroll
    for (int s = 0; s < SPT; s++) ws_dec[((size_t)unit * P + seg) * M + wv * SPT + s] = segdec[s];
  }
}

// ----------------------------------------------------- phase B: scan
// One thread per (unit, four consecutive state elements of one slot row),
// serial over the segments; the loads of a batch of maps are issued before any
// of the batch's stores.  Slot p holds segment p's map on entry (p < P-1) and
// its start state on exit.
template <int DK, int DV, int M>
__global__ void __launch_bounds__(256)
gsa_bf16_scan(float* __restrict__ ws_state, const float* __restrict__ ws_dec,
              const float* __restrict__ k0, const float* __restrict__ v0, int units, int P) {
  constexpr int NE = M * (DK + DV);
  constexpr int BATCH = 8;
  static_assert(DK % 4 == 0 && DV % 4 == 0, "float4 rows");
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long long)units * (NE / 4)) return;
  const int unit = (int)(gid / (NE / 4)), e = 4 * (int)(gid % (NE / 4));
  const int c = e / (DK + DV), cl = e % (DK + DV);
  f32x4 W = {0.f, 0.f, 0.f, 0.f};
  if (cl < DK) {
    if (k0) W = *reinterpret_cast<const f32x4*>(k0 + ((size_t)unit * M + c) * DK + cl);
  } else {
    if (v0) W = *reinterpret_cast<const f32x4*>(v0 + ((size_t)unit * M + c) * DV + cl - DK);
  }
  f32x4* st = reinterpret_cast<f32x4*>(ws_state + (size_t)unit * P * NE + e);
  const float* dc = ws_dec + (size_t)unit * P * M + c;
  for (int p0 = 0; p0 + 1 < P; p0 += BATCH) {
    f32x4 x[BATCH];
    float d[BATCH];
#pragma unroll
    for (int i = 0; i < BATCH; i++) {
      if (p0 + i + 1 < P) {
        x[i] = st[(size_t)(p0 + i) * (NE / 4)];
        d[i] = dc[(size_t)(p0 + i) * M];
      }
    }
#pragma unroll
    for (int i = 0; i < BATCH; i++) {
      if (p0 + i + 1 < P) {
        __builtin_nontemporal_store(W, st + (size_t)(p0 + i) * (NE / 4));  // read only by the next launch
        W = d[i] * W + x[i];
      }
    }
  }
  __builtin_nontemporal_store(W, st + (size_t)(P - 1) * (NE / 4));
}

// ------------------------------------------------------ phase C: outputs
template <int DK, int DV, int M, int ACT, class Seq>
__global__ void __launch_bounds__(NT, 1)
gsa_bf16_out(const bf16_t* __restrict__ qq, const bf16_t* __restrict__ kk,
             const bf16_t* __restrict__ vv, const bf16_t* __restrict__ gg,
             const float* __restrict__ k0, const float* __restrict__ v0,
             const float* __restrict__ ws_state, bf16_t* __restrict__ oo, float* __restrict__ kf,
             float* __restrict__ vf, const float* __restrict__ ws_dec, Seq seq, int S, int P,
             int units, int fold, float inv_tau, float* __restrict__ lse) {
  using Lds = OutLds<DK, DV, M>;
  using ST = StateTiles<DK, DV, M, 4>;
  // Every wave computes the next chunk's gate factors of GPW slots (after its
  // contractions): an even split measured faster than giving the state waves
  // or the lighter pass waves more of them.
  constexpr int GPW = M / NW;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  bf16_t* sQ = reinterpret_cast<bf16_t*>(smem + Lds::oQ);
  bf16_t* sK = reinterpret_cast<bf16_t*>(smem + Lds::oK);
  bf16_t* sV = reinterpret_cast<bf16_t*>(smem + Lds::oV);
  bf16_t* sW = reinterpret_cast<bf16_t*>(smem + Lds::oW);
  float* sLa = reinterpret_cast<float*>(smem + Lds::oLa);
  float* sDec0 = reinterpret_cast<float*>(smem + Lds::oDec);
  int* sFlag = reinterpret_cast<int*>(smem + Lds::oFlag);
  // factor set b: X, Z, E, dec
  auto fX = [&](int b) { return reinterpret_cast<bf16_t*>(smem + Lds::oF + b * Lds::szF + Lds::fX); };
  auto fZ = [&](int b) { return reinterpret_cast<bf16_t*>(smem + Lds::oF + b * Lds::szF + Lds::fZ); };
  auto fE = [&](int b) { return reinterpret_cast<float*>(smem + Lds::oF + b * Lds::szF + Lds::fE); };
  auto fD = [&](int b) { return reinterpret_cast<float*>(smem + Lds::oF + b * Lds::szF + Lds::fD); };

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const bool is_state = wv >= 4;
  const int sw = wv - 4;
  const int slot0 = wv * GPW;  // this wave's first gate slot
  const SegUnit su = seg_unit(blockIdx.x, P, units, fold);
  const int seg = su.seg, unit = seq.unit_of(su.unit);
  const Span sp = seq.span(unit);
  const int T_len = sp.len;
  const int nchunks = (T_len + C - 1) / C;
  const int c_begin = seg * S, c_end = min(c_begin + S, nchunks);
  // a segment past the end of its sequence (variable-length batches only) has
  // no tokens: it only hands its start state on as the final state when it is
  // the unit's last segment
  const bool empty = Seq::kVar && c_begin >= c_end;
  if (empty && seg != P - 1) return;
  const size_t ub = sp.base;
  const bf16_t* qb = qq + ub * DK;
  const bf16_t* kb = kk + ub * DK;
  const bf16_t* vb = vv + ub * DV;
  constexpr int G = Seq::kGroups, GS = M * G;  // slot groups, gate row pitch
  const int grp = unit % G;
  const bf16_t* gb = gg + gate_base<Seq, M>(sp, unit) + slot0;
  bf16_t* ob = oo + (ub * G + grp) * DV;
  float* lb = G > 1 ? lse + ub * G + grp : nullptr;

  // Gate logits, one row per owner: loaded at the top of a chunk for the next
  // chunk (after the exact path, if this chunk takes it, has read this
  // chunk's row) and used after the contractions, when it has long arrived.
  // (one row type for every wave: rows of two widths here once let the
  // compiler merge their loads into one with a runtime-chosen destination,
  // which put the row in scratch memory)
  typedef GateRow<GPW> Row;
  Row gr;
  auto load_gates = [&](Row& r, int t0, int rv, int lane_) {
    r.load(gb + (size_t)(t0 + min(lane_, rv - 1)) * GS);
  };
  // (the empty asm of pin() keeps the use of the logits, and so the wait for
  // their load, at the call)
  auto factors = [&](Row& r, int rv, int fb, int lane_) -> int {
    r.pin();
    float e_unused[GPW];
    return chunk_factors<GPW, Lds::LDX, Lds::LDE, M>(r, lane_ < rv, inv_tau, lane_, slot0, fX(fb), fZ(fb),
                                                      fE(fb), fD(fb), sDec0 + fb * M, e_unused);
  };
  auto log_alpha = [&](const Row& r, int rv, int lane_) {  // natural log, exact path
#pragma unroll
    for (int s = 0; s < GPW; s++) {
      const float x = r.at(s);
      const float la = (fminf(x, 0.f) - log1pf(__expf(-fabsf(x)))) * inv_tau;
      sLa[lane_ * M + slot0 + s] = lane_ < rv ? la : 0.f;
    }
  };
  auto rows_of = [&](int ch) { return min(C, T_len - ch * C); };

  Tile<DK> pq, pk;
  Tile<DV> pv;
  ST W;
  int regime;  // the current chunk's kNeedSub / kNeedExact bits
  {
    const int t0 = c_begin * C, rv = rows_of(c_begin);
    if (!empty) {
      pq.load(qb + (size_t)t0 * DK, rv, tid);
      pk.load(kb + (size_t)t0 * DK, rv, tid);
      pv.load(vb + (size_t)t0 * DV, rv, tid);
      load_gates(gr, t0, rv, lane);
    }
    if (is_state) {
      if (P > 1 && !fold) {
        W.load_w(ws_state + ((size_t)unit * P + seg) * M * (DK + DV), sw, lane);  // from the scan
      } else {
        W.load_kv(k0 ? k0 + (size_t)unit * M * DK : nullptr, v0 ? v0 + (size_t)unit * M * DV : nullptr, sw, lane);
        // the start state as the segment recurrence over the maps of the
        // segments before this one, one map loading while the last is folded
        if (seg > 0) {
          const float* mp = ws_state + (size_t)unit * P * M * (DK + DV);
          const float* dp = ws_dec + (size_t)unit * P * M;
          constexpr size_t MS = (size_t)M * (DK + DV);
          typename ST::MapRegs xa, xb;
          W.load_map(xa, mp, sw, lane);
          for (int p = 0; p < seg; p += 2) {
            if (p + 1 < seg) W.load_map(xb, mp + (p + 1) * MS, sw, lane);
            W.fold(xa, dp + (size_t)p * M, lane);
            if (p + 1 < seg) {
              if (p + 2 < seg) W.load_map(xa, mp + (p + 2) * MS, sw, lane);
              W.fold(xb, dp + (size_t)(p + 1) * M, lane);
            }
          }
        }
      }
      W.store_copy(sW, Lds::LDW, sw, lane);
    }
    regime = empty ? 0 : block_or(factors(gr, rv, 0, lane), sFlag, 0, lane, wv);
  }

  int b = 0;  // factor set of the current chunk
  for (int ch = c_begin; ch < c_end; ch++) {
    // lane / thread indices re-derived each chunk: keeps the compiler from
    // holding every per-lane LDS address of the loop in registers across it
    int lane_i = lane, tid_i = tid;
    asm volatile("" : "+v"(lane_i), "+v"(tid_i));
    const int t0 = ch * C, rv = rows_of(ch);
    const int cn = min(ch + 1, c_end - 1);  // next chunk (this one again at the end)
    const int t1 = cn * C, rv1 = rows_of(cn);
    pq.store(sQ, Lds::LDQ, rv, tid_i);
    pk.store(sK, Lds::LDQ, rv, tid_i);
    pv.store(sV, Lds::LDV, rv, tid_i);
    const bool slow = regime & kNeedExact;
    if (slow) log_alpha(gr, rv, lane_i);
    load_gates(gr, t1, rv1, lane_i);
    __syncthreads();
    // prefetch the next chunk's tiles into registers (unconditionally -- the
    // last chunk reloads itself -- so that no branch blurs the load-count waits)
    pq.load(qb + (size_t)t1 * DK, rv1, tid_i);
    pk.load(kb + (size_t)t1 * DK, rv1, tid_i);
    pv.load(vb + (size_t)t1 * DV, rv1, tid_i);
    int small;
    if (!slow) {
      if (!is_state) {
        bf16_t* orow = ob + (size_t)t0 * (DV * G);
        float* lrow = G > 1 ? lb + (size_t)t0 * G : nullptr;
        // pass waves hold no state: dropping it frees these registers for the passes
        W.zero();
        const bf16_t* x = fX(b);
        const float* e = fE(b);
        const float* d = fD(b);
        if (!(regime & kNeedSub)) {
          switch (wv) {
            case 0: pass_chunk<DK, DV, M, 0, ACT, G, false>(lane_i, sQ, sK, sV, sW, x, e, d, orow, lrow, rv); break;
            case 1: pass_chunk<DK, DV, M, 1, ACT, G, false>(lane_i, sQ, sK, sV, sW, x, e, d, orow, lrow, rv); break;
            case 2: pass_chunk<DK, DV, M, 2, ACT, G, false>(lane_i, sQ, sK, sV, sW, x, e, d, orow, lrow, rv); break;
            default: pass_chunk<DK, DV, M, 3, ACT, G, false>(lane_i, sQ, sK, sV, sW, x, e, d, orow, lrow, rv); break;
          }
        } else {  // some slot decays out of the chunk form's range: sub-chunk reference points
          switch (wv) {
            // rows of sub-chunk 0: its reference point is the chunk start, so
            // the sub-chunk form is the plain one
            case 0: pass_chunk<DK, DV, M, 0, ACT, G, false>(lane_i, sQ, sK, sV, sW, x, e, d, orow, lrow, rv); break;
            case 1: pass_chunk<DK, DV, M, 1, ACT, G, true>(lane_i, sQ, sK, sV, sW, x, e, d, orow, lrow, rv); break;
            case 2: pass_chunk<DK, DV, M, 2, ACT, G, true>(lane_i, sQ, sK, sV, sW, x, e, d, orow, lrow, rv); break;
            default: pass_chunk<DK, DV, M, 3, ACT, G, true>(lane_i, sQ, sK, sV, sW, x, e, d, orow, lrow, rv); break;
          }
        }
      } else {
        W.carry(sK, Lds::LDQ, sV, Lds::LDV, fZ(b), Lds::LDX, sDec0 + b * M, sw, lane_i);
      }
      // the next chunk's factors
      small = factors(gr, rv1, b ^ 1, lane_i);
    } else {
      // ---- exact token recurrence (no division by a decay product), on an
      // fp32 copy of the state in LDS; thread t owns slot t / TPS and 1/TPS of
      // its columns for the whole chunk
      exact_chunk<DK, DV, M, ACT, G>(W, rv, smem, sQ, sK, sV, ob + (size_t)t0 * (DV * G),
                                     G > 1 ? lb + (size_t)t0 * G : nullptr, tid_i);
      small = factors(gr, rv1, b ^ 1, lane_i);
    }
    regime = block_or(small, sFlag, ch - c_begin + 1, lane_i, wv);
    if (is_state) W.store_copy(sW, Lds::LDW, sw, lane_i);
    b ^= 1;
  }

  if (seg == P - 1 && is_state)
    W.store_kv(kf ? kf + (size_t)unit * M * DK : nullptr, vf ? vf + (size_t)unit * M * DV : nullptr, sw, lane);
}

// ------------------------------------------------------ slot-group merge
// The read of 2M slots from the two groups' normalised outputs o_h and
// log-sum-exps l_h (SlotGroups).  The softmax over all the slots weighs group
// h by w_h = exp(l_h - L), L = log(exp(l_0) + exp(l_1)), so o = w_0 o_0 +
// w_1 o_1 (Sec. 3.2, the softmax read); an element-wise read adds the groups.
// part [rows][2][DV] bf16, lse [rows][2] fp32.  Thread = 8 columns of one
// token row.
template <int DV, bool SOFTMAX>
__global__ void __launch_bounds__(256)
gsa_bf16_merge(const bf16_t* __restrict__ part, const float* __restrict__ lse, bf16_t* __restrict__ o,
               size_t rows) {
  constexpr int TPR = DV / 8;  // threads per row, a power of two dividing a wave
  static_assert(DV % 8 == 0 && 64 % TPR == 0, "row width");
  const size_t gid = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t row = gid / TPR;
  const int c = (int)(gid % TPR) * 8;
  if (row >= rows) return;
  float w0 = 1.f, w1 = 1.f;
  if constexpr (SOFTMAX) {
    const float2 l = *reinterpret_cast<const float2*>(lse + 2 * row);
    const float mx = fmaxf(l.x, l.y);
    const float e0 = __expf(l.x - mx), e1 = __expf(l.y - mx);
    const float inv = 1.f / (e0 + e1);
    w0 = e0 * inv;
    w1 = e1 * inv;
  }
  const uint4 a = *reinterpret_cast<const uint4*>(part + (2 * row) * DV + c);
  const uint4 b = *reinterpret_cast<const uint4*>(part + (2 * row + 1) * DV + c);
  const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
  float r[8];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    r[2 * i] = w0 * __uint_as_float(aw[i] << 16) + w1 * __uint_as_float(bw[i] << 16);
    r[2 * i + 1] = w0 * __uint_as_float(aw[i] & 0xffff0000u) + w1 * __uint_as_float(bw[i] & 0xffff0000u);
  }
  uint32_t ow[4];
#pragma unroll
  for (int i = 0; i < 4; i++) ow[i] = (uint32_t)f2bf(r[2 * i]) | ((uint32_t)f2bf(r[2 * i + 1]) << 16);
  __builtin_nontemporal_store(u32x4{ow[0], ow[1], ow[2], ow[3]}, reinterpret_cast<u32x4*>(o + row * DV + c));
}

// ------------------------------------------------------------ launcher
// a.T is the sequence length (dense) or the longest one (variable-length);
// the segment count P follows from it, and the segments of shorter sequences
// past their end are empty.
template <int DK, int DV, int M, int ACT, class Seq>
static int launch(const GsaLaunch& a, const Seq& seq) {
  using LO = OutLds<DK, DV, M>;
  using LS = StateLds<DK, DV, M>;
  const int units = a.B * a.H;
  const int nchunks = (a.T + C - 1) / C;
  const int S = a.chunks_per_seg;
  const int P = (nchunks + S - 1) / S;
  const float inv_tau = 1.0f / a.tau;
  hipStream_t st = (hipStream_t)a.stream;
  static const bool lds_set = [] {  // once per instantiation and process
    (void)hipFuncSetAttribute((const void*)gsa_bf16_out<DK, DV, M, ACT, Seq>,
                        hipFuncAttributeMaxDynamicSharedMemorySize, LO::total);
    (void)hipFuncSetAttribute((const void*)gsa_bf16_state<DK, DV, M, Seq>,
                        hipFuncAttributeMaxDynamicSharedMemorySize, LS::total);
    return true;
  }();
  (void)lds_set;
  // With few segments the output workgroups fold the maps of the segments
  // before theirs into their start state themselves: that costs the last
  // segment's workgroup P - 1 map reads, all through one CU, and saves the scan
  // launch and its wait (measured: a gain at 1 and 3 maps, a loss at 7).  Every
  // output workgroup then reads k0 / v0, so not when the final state is written
  // over them (the last segment could finish before another one has started).
  const bool in_place = (a.kf && a.kf == a.k0) || (a.vf && a.vf == a.v0);
  const bool keep = a.keep_states != nullptr;
  const int fold = !keep && P > 1 && P - 1 <= kMaxFoldedMaps && !in_place;
  if (P > 1) {
    launch_timed(gsa_bf16_state<DK, DV, M, Seq>, dim3(P - 1, units), dim3(NT), LS::total, a.stream,
                 a.events, 0, 1, (const bf16_t*)a.k, (const bf16_t*)a.v, (const bf16_t*)a.g,
                 a.ws_state, a.ws_dec, seq, S, P, inv_tau);
    if (!fold) {
      const long long ne = (long long)units * M * (DK + DV) / 4;  // float4 per thread
      hipLaunchKernelGGL((gsa_bf16_scan<DK, DV, M>), dim3((unsigned)((ne + 255) / 256)), dim3(256), 0, st,
                         a.ws_state, (const float*)a.ws_dec, a.k0, a.v0, units, P);
    }
  } else {
    record_event(a.events, 0, a.stream);
    record_event(a.events, 1, a.stream);
    if (keep) {  // one segment: its start state is the initial state
      const long long ne = (long long)units * M * (DK + DV) / 4;
      hipLaunchKernelGGL((gsa_bf16_scan<DK, DV, M>), dim3((unsigned)((ne + 255) / 256)), dim3(256), 0, st,
                         a.ws_state, (const float*)a.ws_dec, a.k0, a.v0, units, P);
    }
  }
  launch_timed(gsa_bf16_out<DK, DV, M, ACT, Seq>, dim3(P * units), dim3(NT), LO::total, a.stream,
               a.events, 2, 3, (const bf16_t*)a.q, (const bf16_t*)a.k, (const bf16_t*)a.v,
               (const bf16_t*)a.g, a.k0, a.v0, (const float*)a.ws_state, (bf16_t*)a.o, a.kf, a.vf,
               (const float*)a.ws_dec, seq, S, P, units, fold, inv_tau, a.ws_lse);
  return 0;
}

// 2M slots as two groups of M (SlotGroups): the group launches over 2BH units
// (a.chunks_per_seg and the workspace sized for them), then the merge.
template <int DK, int DV, int M, int ACT>
static int launch_groups(const GsaLaunch& a) {
  GsaLaunch b = a;
  b.H = 2 * a.H;
  b.o = a.ws_part;
  if (launch<DK, DV, M, ACT, SlotGroups>(b, SlotGroups{a.T}) != 0) return -1;
  const size_t rows = (size_t)a.B * a.H * a.T;
  const size_t threads = rows * (DV / 8);
  hipLaunchKernelGGL((gsa_bf16_merge<DV, ACT == kActSoftmax>), dim3((unsigned)((threads + 255) / 256)),
                     dim3(256), 0, (hipStream_t)a.stream, (const bf16_t*)a.ws_part, (const float*)a.ws_lse,
                     (bf16_t*)a.o, rows);
  return 0;
}

template <int DK, int DV, int M>
static int launch_act_groups(const GsaLaunch& a) {
  if (a.cu_seqlens || !a.ws_part || !a.ws_lse) return -1;
  switch (a.act) {
    case kActSoftmax: return launch_groups<DK, DV, M, kActSoftmax>(a);
    case kActIdentity: return launch_groups<DK, DV, M, kActIdentity>(a);
    case kActSwish: return launch_groups<DK, DV, M, kActSwish>(a);
    case kActRelu: return launch_groups<DK, DV, M, kActRelu>(a);
    case kActRelu2: return launch_groups<DK, DV, M, kActRelu2>(a);
    default: return -1;
  }
}

template <int DK, int DV, int M>
static int launch_act(const GsaLaunch& a) {
  if (a.cu_seqlens) {  // packed variable-length batch: the softmax read only
    if (a.act != kActSoftmax || a.n_seqs < 0) return -1;
    // Groups of at most kMaxVarSeqs sequences, one launch sequence each (a
    // group's offsets travel in the kernel arguments); the groups run one
    // after the other on the stream and share the workspace.
    const int groups = (a.n_seqs + kMaxVarSeqs - 1) / kMaxVarSeqs;
    if (groups > 1) {
      record_event(a.events, 0, a.stream);
      record_event(a.events, 1, a.stream);
    }
    const size_t MK = (size_t)a.H * M * DK, MV = (size_t)a.H * M * DV;
    for (int g0 = 0; g0 < a.n_seqs; g0 += kMaxVarSeqs) {
      const int ng = min(kMaxVarSeqs, a.n_seqs - g0);
      VarSeqs vs{};
      vs.H = a.H;
      vs.total = a.cu_seqlens[a.n_seqs];
      int tmax = 0;
      for (int i = 0; i <= ng; i++) vs.cu[i] = a.cu_seqlens[g0 + i];
      for (int i = 0; i < ng; i++) tmax = max(tmax, vs.cu[i + 1] - vs.cu[i]);
      GsaLaunch b = a;
      b.B = ng;
      b.T = tmax;
      b.k0 = a.k0 ? a.k0 + g0 * MK : nullptr;
      b.v0 = a.v0 ? a.v0 + g0 * MV : nullptr;
      b.kf = a.kf ? a.kf + g0 * MK : nullptr;
      b.vf = a.vf ? a.vf + g0 * MV : nullptr;
      b.events = groups == 1 ? a.events : nullptr;
      if (tmax == 0) {  // only empty sequences: the final states are the initial ones
        state_copy(b.kf, b.k0, (size_t)ng * MK, a.stream);
        state_copy(b.vf, b.v0, (size_t)ng * MV, a.stream);
        for (int e = 0; e < 4; e++) record_event(b.events, e, a.stream);  // only with one group
        continue;
      }
      // longest first (stable: equal lengths keep their order, so equal-length
      // batches launch exactly like the dense one)
      for (int i = 0; i < ng; i++) vs.order[i] = i;
      std::stable_sort(vs.order, vs.order + ng, [&](int x, int y) {
        return vs.cu[x + 1] - vs.cu[x] > vs.cu[y + 1] - vs.cu[y];
      });
      if (launch<DK, DV, M, kActSoftmax, VarSeqs>(b, vs) != 0) return -1;
    }
    if (groups > 1) {
      record_event(a.events, 2, a.stream);
      record_event(a.events, 3, a.stream);
    }
    return 0;
  }
  const DenseSeqs ds{a.T};
  switch (a.act) {
    case kActSoftmax: return launch<DK, DV, M, kActSoftmax>(a, ds);
    case kActIdentity: return launch<DK, DV, M, kActIdentity>(a, ds);
    case kActSwish: return launch<DK, DV, M, kActSwish>(a, ds);
    case kActRelu: return launch<DK, DV, M, kActRelu>(a, ds);
    case kActRelu2: return launch<DK, DV, M, kActRelu2>(a, ds);
    default: return -1;
  }
}

}  // namespace bfk

namespace bfk {
// The segment start states of a dense batch, as the forward computes them:
// state maps of segments 0 .. P-2 and the per-unit scan, so that ws_state[u][p]
// (layout [units][P][M][DK+DV] fp32) holds the state at the start of segment p
// (p = 0: the initial state).  ws_dec: [units][P][M] fp32.
template <int DK, int DV, int M, class Seq>
static void segment_states(const void* k, const void* v, const void* g, const float* k0,
                           const float* v0, float* ws_state, float* ws_dec, int units, int T, int S,
                           int P, float tau, void* stream) {
  using LS = StateLds<DK, DV, M>;
  static const bool lds_set = [] {
    (void)hipFuncSetAttribute((const void*)gsa_bf16_state<DK, DV, M, Seq>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, LS::total);
    return true;
  }();
  (void)lds_set;
  hipStream_t st = (hipStream_t)stream;
  if (P > 1)
    hipLaunchKernelGGL((gsa_bf16_state<DK, DV, M, Seq>), dim3(P - 1, units), dim3(NT), LS::total, st,
                       (const bf16_t*)k, (const bf16_t*)v, (const bf16_t*)g, ws_state, ws_dec,
                       Seq{T}, S, P, 1.0f / tau);
  const long long ne = (long long)units * M * (DK + DV) / 4;
  hipLaunchKernelGGL((gsa_bf16_scan<DK, DV, M>), dim3((unsigned)((ne + 255) / 256)), dim3(256), 0, st,
                     ws_state, (const float*)ws_dec, k0, v0, units, P);
}
}  // namespace bfk

int gsa_bf16_segment_states(int dk, int dv, int m, int groups, const void* k, const void* v, const void* g,
                            const float* k0, const float* v0, float* ws_state, float* ws_dec,
                            int units, int T, int S, int P, float tau, void* stream) {
#define SEG_CASE(DKC, DVC, MC)                                                                        \
  if (dk == DKC && dv == DVC && m == MC) {                                                            \
    if (groups == 2)                                                                                  \
      bfk::segment_states<DKC, DVC, MC, bfk::SlotGroups>(k, v, g, k0, v0, ws_state, ws_dec, units, T, \
                                                         S, P, tau, stream);                          \
    else                                                                                              \
      bfk::segment_states<DKC, DVC, MC, bfk::DenseSeqs>(k, v, g, k0, v0, ws_state, ws_dec, units, T,  \
                                                        S, P, tau, stream);                           \
    return 0;                                                                                         \
  }
  if (groups != 1 && !(groups == 2 && m == 64)) return -1;
  SEG_CASE(128, 128, 64)
  SEG_CASE(128, 128, 32)
  SEG_CASE(64, 64, 64)
  SEG_CASE(64, 64, 32)
#undef SEG_CASE
  return -1;
}

#define GSA_BF16_CASE(DKC, DVC, MC)                                      \
  if (dk == DKC && dv == DVC && m == MC) {                                \
    static_assert(bfk::OutLds<DKC, DVC, MC>::total <= kLdsBytes, "LDS"); \
    if (query) return bfk::OutLds<DKC, DVC, MC>::total;                   \
    return bfk::launch_act<DKC, DVC, MC>(*a);                             \
  }

// m = 2M as two slot groups of M (slot_groups(1, m) == 2)
#define GSA_BF16_GROUPS_CASE(DKC, DVC, MC)                                \
  if (dk == DKC && dv == DVC && m == 2 * MC) {                            \
    if (query) return bfk::OutLds<DKC, DVC, MC>::total;                   \
    return bfk::launch_act_groups<DKC, DVC, MC>(*a);                      \
  }

// Returns: query -> LDS bytes (>0) or -1 if unsupported; launch -> 0 or -1.
int gsa_dispatch_bf16(int dk, int dv, int m, const GsaLaunch* a, bool query) {
  GSA_BF16_GROUPS_CASE(128, 128, 64)
  GSA_BF16_GROUPS_CASE(64, 64, 64)
  GSA_BF16_CASE(128, 128, 64)
  GSA_BF16_CASE(128, 128, 32)
  GSA_BF16_CASE(64, 64, 64)
  GSA_BF16_CASE(64, 64, 32)
  return -1;
}

}  // namespace gsa
