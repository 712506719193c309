// Chunkwise gated linear attention (GLA) forward on gfx950, bf16 inputs, fp32
// state and accumulation.
//
// Method: "Gated Slot Attention for Efficient Linear-Time Sequence Modeling"
// (arXiv 2409.07146), Sec. 2.3 (GLA with beta = 1):
//   S_t = Diag(alpha_t) S_{t-1} + k_t v_t^T,  o_t = S_t^T q_t,
//   alpha_t = sigmoid(g_t)^(1/tau) per key dimension, S in R^{dk x dv},
// and App. A.1 (chunk form: a read of the chunk-start state plus a causal
// intra-chunk term).  Per chunk of C = 64 tokens, with the chunk-local
// E_j = prod_{i<=j} alpha_i per key dimension:
//   Qt = Q * E,  Kt = K / E                                  [C x dk]
//   O   = Qt S_0 + mask(Qt Kt^T) V                           [C x dv]
//   S^T <- (S_0^T + V^T Kt) Diag(E_C)                        [dv x dk]
// The outputs are computed transposed (O^T = S_0^T Qt^T + V^T mask(Kt Qt^T))
// so that the masked score block leaves the matrix cores in the register
// layout the value contraction takes as an operand.
//
// Launches (no inter-workgroup waiting), as for the GSA forward: state maps of
// sub-segments (gla_bf16_state, from a zero start, in the overflow-free form
// S^T <- S^T Diag(E_C) + V^T (K * E_C / E)), an fp32 scan that turns them into
// the start state of every output segment (gla_bf16_scan), and the outputs
// (gla_bf16_out).  The state-map pass may split each output segment into
// several sub-segments so that it fills the chip when there are few
// (batch, head) units.  With at most kMaxFoldedMaps maps before the last
// segment the output workgroups fold them into their start states themselves
// and there is no scan launch.
//
// Output kernel, per workgroup of 512 threads:
//   waves 0..3 ("pass"): token rows 16J..16J+15 of the chunk (J = wave);
//   waves 4..7 ("state"): S^T in MFMA accumulators (a quarter each) and the
//              bf16 copy of S the pass waves read;
//   all waves: the next chunk's factors Qt, Kt, E_C (key dimensions
//              [DK/8 w, DK/8 (w+1)) of every token, token = lane, so that the
//              cumulative decay is a wave-wide prefix sum), into the second of
//              two factor sets: the state waves before the chunk's first
//              barrier (beside the pass waves' contractions), the pass waves
//              after it (beside the state copy).
// A chunk whose decay product falls below 2^-90 in some key dimension runs as
// the exact token recurrence instead (no division by a decay product).
#include "bf16_common.hpp"
#include "common.hpp"
#include "internal.hpp"
#include "launch.hpp"

namespace gsa {
namespace bfk {

// --------------------------------------------------------------- LDS plans
template <int DK, int DV>
struct GlaOutLds {
  static constexpr int PAD = 8;
  static constexpr int LDQ = DK + PAD, LDV = DV + PAD, LDS = DV + PAD;
  // V tile of the current chunk (staged one chunk ahead, after the barrier
  // that ends its readers)
  static constexpr int szV = C * LDV * 2;
  static constexpr int oV = 0;
  // factor set b: Qt, Kt [C][LDQ] bf16 (raw q, k until the factor step turns
  // them into Qt, Kt in place); the bf16 copy of S [DK][LDS] sits between the
  // two sets so that either set and the copy form one contiguous region
  static constexpr int szQK = 2 * C * LDQ * 2;
  static constexpr int oF0 = szV;
  static constexpr int oS = oF0 + szQK;
  static constexpr int oF1 = oS + DK * LDS * 2;
  static constexpr int fQ = 0, fK = C * LDQ * 2;
  static constexpr int oEc = oF1 + szQK;                 // 2 x [DK] fp32
  static constexpr int szG = C * LDQ * 2;                // raw gate logits [C][LDQ] bf16
  static constexpr int oG0 = oEc + 2 * DK * 4;           // of set 0, then of set 1
  static constexpr int oFlag = oG0 + 2 * szG;            // 2 x NW ints
  static constexpr int total = oFlag + 2 * NW * 4;
  // exact path, inside [set b | copy of S] (b = 0) or [copy of S | set 1]
  // (b = 1): fp32 S [DK][DV] for the change of layout, then (after it was
  // read) raw q, k, g tiles [C][DK] bf16 and output partials [NW][DV] fp32
  static constexpr int szR = szQK + DK * LDS * 2;
  static constexpr int xSf = 0, xQr = 0, xKr = C * DK * 2, xGr = 2 * C * DK * 2, xOp = 3 * C * DK * 2;
  static_assert(DK * DV * 4 <= szR && xOp + NW * DV * 4 <= szR, "exact path must fit its region");
  __device__ __forceinline__ static int oF(int b) { return b ? oF1 : oF0; }
  __device__ __forceinline__ static int oG(int b) { return oG0 + b * szG; }
  __device__ __forceinline__ static int oX(int b) { return b ? oS : oF0; }
  static_assert(szV % 16 == 0 && szQK % 16 == 0 && oS % 16 == 0 && oF1 % 16 == 0 && oEc % 16 == 0 &&
                    oG0 % 16 == 0 && szG % 16 == 0 && oFlag % 16 == 0 && xKr % 16 == 0 &&
                    xGr % 16 == 0 && xOp % 16 == 0,
                "LDS tiles must stay 16-byte aligned");
};

template <int DK, int DV>
struct GlaStateLds {  // two buffers of everything a chunk needs (software pipeline)
  static constexpr int PAD = 8;
  static constexpr int LDQ = DK + PAD, LDV = DV + PAD;
  static constexpr int oK = 0;
  static constexpr int oV = oK + C * LDQ * 2;
  static constexpr int oEc = oV + C * LDV * 2;
  static constexpr int szBuf = oEc + DK * 4;
  static constexpr int total = 2 * szBuf;
  static_assert(oV % 16 == 0 && oEc % 16 == 0 && szBuf % 16 == 0, "alignment");
};

// ------------------------------------------------------------ state tiles
// S^T [DV x DK] in MFMA accumulators held by NSW waves.  The 16x16 tiles form
// two column blocks (key dimensions) and NSW/2 row blocks (value dimensions);
// wave sw owns row block sw/2 and column block sw%2: NA x NB tiles.  Lane l of
// tile (a, b) holds S^T[16 n(a) + 4(l/16) + i][16 c(b) + l%16], i = 0..3.
template <int DK, int DV, int NSW>
struct GlaTiles {
  static constexpr int NTN = DV / 16, NTC = DK / 16;
  static constexpr int NB = NTC / 2;
  static constexpr int NA = 2 * NTN / NSW;
  static_assert(NTC % 2 == 0 && (2 * NTN) % NSW == 0 && NA >= 1, "state tiles must split evenly");
  f32x4 st[NA][NB];

  __device__ __forceinline__ static int n_of(int sw, int a) { return 16 * ((sw >> 1) * NA + a); }
  __device__ __forceinline__ static int c_of(int sw, int b) { return 16 * ((sw & 1) * NB + b); }

  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int a = 0; a < NA; a++)
#pragma unroll
      for (int b = 0; b < NB; b++) st[a][b] = zero4();
  }
  // S [DK][DV] fp32 row-major (ld = row length), nullable (zeros)
  __device__ __forceinline__ void load(const float* __restrict__ S, int ld, int sw, int lane) {
    const int L = lane & 15, g = lane >> 4;
#pragma unroll
    for (int a = 0; a < NA; a++)
#pragma unroll
      for (int b = 0; b < NB; b++) {
        if (S) {
          const float4 x = *reinterpret_cast<const float4*>(S + (size_t)(c_of(sw, b) + L) * ld + n_of(sw, a) + 4 * g);
          st[a][b] = f32x4{x.x, x.y, x.z, x.w};
        } else {
          st[a][b] = zero4();
        }
      }
  }
  __device__ __forceinline__ void store(float* __restrict__ S, int ld, int sw, int lane) const {
    const int L = lane & 15, g = lane >> 4;
#pragma unroll
    for (int a = 0; a < NA; a++)
#pragma unroll
      for (int b = 0; b < NB; b++)
        *reinterpret_cast<float4*>(S + (size_t)(c_of(sw, b) + L) * ld + n_of(sw, a) + 4 * g) =
            make_float4(st[a][b][0], st[a][b][1], st[a][b][2], st[a][b][3]);
  }
  // one sub-segment map (layout of load) into registers, and the segment step
  // S <- Diag(dec) S + map (rows = key dimensions) with the scan kernel's
  // operation order
  typedef f32x4 MapRegs[NA][NB];
  __device__ __forceinline__ void load_map(MapRegs& x, const float* __restrict__ S, int sw, int lane) const {
    const int L = lane & 15, g = lane >> 4;
#pragma unroll
    for (int a = 0; a < NA; a++)
#pragma unroll
      for (int b = 0; b < NB; b++) {
        const float4 v = *reinterpret_cast<const float4*>(S + (size_t)(c_of(sw, b) + L) * DV + n_of(sw, a) + 4 * g);
        x[a][b] = f32x4{v.x, v.y, v.z, v.w};
      }
  }
  __device__ __forceinline__ void fold(const MapRegs& x, const float* __restrict__ dec, int sw, int lane) {
#pragma unroll
    for (int b = 0; b < NB; b++) {
      const float d = dec[c_of(sw, b) + (lane & 15)];
#pragma unroll
      for (int a = 0; a < NA; a++)
#pragma unroll
        for (int i = 0; i < 4; i++) st[a][b][i] = d * st[a][b][i] + x[a][b][i];
    }
  }
  // bf16 copy of S, row-major [DK][ld]
  __device__ __forceinline__ void store_copy(bf16_t* sS, int ld, int sw, int lane) const {
    const int L = lane & 15, g = lane >> 4;
#pragma unroll
    for (int a = 0; a < NA; a++)
#pragma unroll
      for (int b = 0; b < NB; b++)
        *reinterpret_cast<bf16x4v*>(sS + (c_of(sw, b) + L) * ld + n_of(sw, a) + 4 * g) = pack4(st[a][b]);
  }
  // one chunk: S^T += V^T Kx over the chunk's tokens, with the column scaling
  // by E_C (sEc) applied after (POST, Kx = K / E) or before (!POST,
  // Kx = K * E_C / E) the accumulation
  template <bool POST>
  __device__ __forceinline__ void carry(const bf16_t* sV, int ldv, const bf16_t* sKx, int ldk,
                                        const float* sEc, int sw, int lane) {
    const int L = lane & 15, g = lane >> 4;
    float ec[NB];
#pragma unroll
    for (int b = 0; b < NB; b++) ec[b] = sEc[c_of(sw, b) + L];
    if constexpr (!POST) scale(ec);
#pragma unroll
    for (int r0 = 0; r0 < C; r0 += 32) {
      bf16x8 va[NA], kb[NB];
#pragma unroll
      for (int a = 0; a < NA; a++) va[a] = ld_col(sV, ldv, n_of(sw, a), r0 + 8 * g, r0 + 8 * g + 4, lane);
#pragma unroll
      for (int b = 0; b < NB; b++) kb[b] = ld_col(sKx, ldk, c_of(sw, b), r0 + 8 * g, r0 + 8 * g + 4, lane);
#pragma unroll
      for (int a = 0; a < NA; a++)
#pragma unroll
        for (int b = 0; b < NB; b++) st[a][b] = mma(va[a], kb[b], st[a][b]);
    }
    if constexpr (POST) scale(ec);
  }
  __device__ __forceinline__ void scale(const float (&ec)[NB]) {
#pragma unroll
    for (int a = 0; a < NA; a++)
#pragma unroll
      for (int b = 0; b < NB; b++)
#pragma unroll
        for (int i = 0; i < 4; i++) st[a][b][i] *= ec[b];
  }
};

// -------------------------------------------------------- chunk factors
// Key dimensions d0..d0+SPT-1 of one chunk, token row = lane (rows >= rv are
// identity steps): G = chunk-local cumulative log2 alpha.  Output-pass form,
// from the raw q, k, g rows staged in LDS: Qt = q exp2(G) and Kt = k exp2(-G)
// (0 on rows >= rv), written over q and k, and E_C = exp2(G_C).  Returns
// whether any of these dimensions decays below the range of the factorised
// form in this chunk.
template <int SPT, int LDQ, int GM>
__device__ __forceinline__ bool out_factors(bf16_t* sQ, bf16_t* sK, const bf16_t* sG, int rv,
                                            float inv_tau, int lane, int d0, float* sEc) {
  const bool valid = lane < rv;
  float q[SPT], k[SPT], G[SPT];
  lds_row<SPT>(sQ + lane * LDQ + d0, q);
  lds_row<SPT>(sK + lane * LDQ + d0, k);
  lds_row<SPT>(sG + lane * LDQ + d0, G);
#pragma unroll
  for (int s = 0; s < SPT; s++) G[s] = gate_log2_mode<GM>(G[s], valid, inv_tau);
  wave_prefix_sums<SPT>(G);
  bool small = false;
  float ec[SPT];
#pragma unroll
  for (int s = 0; s < SPT; s++) {
    const float gc = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(G[s]), 63));
    small |= !(gc >= kFastMinLog2Decay);
    const float e = __builtin_amdgcn_exp2f(G[s]);
    ec[s] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(e), 63));
    q[s] *= e;
    k[s] = (valid ? k[s] : 0.f) * __builtin_amdgcn_exp2f(-G[s]);
  }
  store_bf16_row<SPT>(sQ + lane * LDQ + d0, q);
  store_bf16_row<SPT>(sK + lane * LDQ + d0, k);
  if (lane == 0) store_f32_row<SPT>(sEc + d0, ec);
  return small;
}

// State-map form (any decay): Kh = k exp2(G_C - G) (0 on rows >= rv) and
// E_C = exp2(G_C), which also multiplies into the running decay product.
template <int SPT, int LDQ, int GM>
__device__ __forceinline__ void map_factors(const GateRow<SPT>& k, const GateRow<SPT>& g, int rv,
                                            float inv_tau, int lane, int d0, bf16_t* sKh, float* sEc,
                                            float (&dec)[SPT], bool count) {
  const bool valid = lane < rv;
  float G[SPT];
#pragma unroll
  for (int s = 0; s < SPT; s++) G[s] = gate_log2_mode<GM>(g.at(s), valid, inv_tau);
  wave_prefix_sums<SPT>(G);
  float kh[SPT], ec[SPT];
#pragma unroll
  for (int s = 0; s < SPT; s++) {
    const float gc = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(G[s]), 63));
    ec[s] = __builtin_amdgcn_exp2f(gc);
    kh[s] = (valid ? k.at(s) : 0.f) * __builtin_amdgcn_exp2f(gc - G[s]);
    dec[s] *= count ? ec[s] : 1.f;
  }
  store_bf16_row<SPT>(sKh + lane * LDQ + d0, kh);
  if (lane == 0) store_f32_row<SPT>(sEc + d0, ec);
}

// -------------------------------------------------------- pass-wave chunk
// Token rows 16J..16J+15: scores A^T = mask(Kt Qt^T) for row tiles R <= J,
// then O^T = S^T Qt^T + V^T A^T in groups of four value-column tiles, stored as
// 8-byte row pieces.  Reads sQt, sKt, sV and the bf16 state copy sS.
template <int DK, int DV, int J>
__device__ __forceinline__ void gla_pass_chunk(int lane, const bf16_t* sQt, const bf16_t* sKt,
                                               const bf16_t* sV, const bf16_t* sS,
                                               bf16_t* __restrict__ orow, int rv) {
  using Lds = GlaOutLds<DK, DV>;
  constexpr int KQ = DK / 32, NVT = DV / 16;
  constexpr int NR = J + 1, NPR = J / 2 + 1;
  const int L = lane & 15, g = lane >> 4;
  const int j = 16 * J + L;

  bf16x8 qf[KQ];  // B[c][j] = Qt[j][c]
#pragma unroll
  for (int s = 0; s < KQ; s++) qf[s] = ld_row(sQt, Lds::LDQ, 16 * J, 32 * s, lane);
  f32x4 at[4];
#pragma unroll
  for (int R = 0; R < 4; R++) at[R] = zero4();
#pragma unroll
  for (int s = 0; s < KQ; s++)
#pragma unroll
    for (int R = 0; R < NR; R++) at[R] = mma(ld_row(sKt, Lds::LDQ, 16 * R, 32 * s, lane), qf[s], at[R]);
#pragma unroll
  for (int i = 0; i < 4; i++)
    if (4 * g + i > L) at[J][i] = 0.f;
  bf16x8 af[2];
  af[0] = pack8(at[0], at[1]);
  af[1] = pack8(at[2], at[3]);

  const bool store = j < rv;
  constexpr int NG = NVT < 4 ? NVT : 4;
#pragma unroll
  for (int n0 = 0; n0 < NVT; n0 += NG) {
    f32x4 acc[NG];
#pragma unroll
    for (int u = 0; u < NG; u++) acc[u] = zero4();
#pragma unroll
    for (int s = 0; s < KQ; s++)
#pragma unroll
      for (int u = 0; u < NG; u++)  // A[n][c] = S[c][n]
        acc[u] = mma(ld_col(sS, Lds::LDS, 16 * (n0 + u), 32 * s + 8 * g, 32 * s + 8 * g + 4, lane), qf[s],
                     acc[u]);
#pragma unroll
    for (int pr = 0; pr < NPR; pr++)
#pragma unroll
      for (int u = 0; u < NG; u++)
        acc[u] = mma(ld_col(sV, Lds::LDV, 16 * (n0 + u), 32 * pr + 4 * g, 32 * pr + 16 + 4 * g, lane),
                     af[pr], acc[u]);
    if (store) {
#pragma unroll
      for (int u = 0; u < NG; u++)
        *reinterpret_cast<bf16x4v*>(orow + (size_t)j * DV + 16 * (n0 + u) + 4 * g) = pack4(acc[u]);
    }
  }
}

// ------------------------------------------------ exact chunk recurrence
// One chunk token by token (Sec. 2.3 recurrent form) on an fp32 copy of the
// state: thread t owns key dimension t / TPD and DV / TPD of its value columns.
// The state waves' accumulators go through LDS to and from that layout.
// Contains workgroup barriers: all threads call it.
template <int DK, int DV, int GM>
__device__ __forceinline__ void gla_exact_chunk(GlaTiles<DK, DV, 4>& W, int rv, unsigned char* region,
                                                const bf16_t* sV, const bf16_t* __restrict__ qc,
                                                const bf16_t* __restrict__ kc,
                                                const bf16_t* __restrict__ gc,
                                                bf16_t* __restrict__ orow, int tid, float inv_tau) {
  using Lds = GlaOutLds<DK, DV>;
  constexpr int TPD = NT / DK;  // threads per key dimension
  constexpr int CPT = DV / TPD;  // value columns per thread
  static_assert(NT % DK == 0 && TPD <= 64 && CPT >= 1, "exact-path thread map");
  float* sSf = reinterpret_cast<float*>(region + Lds::xSf);
  bf16_t* sQr = reinterpret_cast<bf16_t*>(region + Lds::xQr);
  bf16_t* sKr = reinterpret_cast<bf16_t*>(region + Lds::xKr);
  bf16_t* sGr = reinterpret_cast<bf16_t*>(region + Lds::xGr);
  float* sOp = reinterpret_cast<float*>(region + Lds::xOp);
  const int lane = tid & 63, wv = tid >> 6;
  const bool is_state = wv >= 4;
  const int d = tid / TPD, p = tid % TPD;

  // (the region held this chunk's factor set and the bf16 state copy, all of
  // whose readers passed the last barrier; the other set holds the next
  // chunk's staged rows and is left alone)
  if (is_state) W.store(sSf, DV, wv - 4, lane);
  __syncthreads();
  float s[CPT];
#pragma unroll
  for (int i = 0; i < CPT; i++) s[i] = sSf[d * DV + p * CPT + i];
  __syncthreads();
  // this chunk's raw q, k, g rows into the same region
  constexpr int VPR = DK / 8;
  for (int idx = tid; idx < C * VPR; idx += NT) {
    const int row = idx / VPR, cv = idx % VPR;
    if (row < rv) {
      *reinterpret_cast<uint4*>(sQr + row * DK + cv * 8) = *reinterpret_cast<const uint4*>(qc + (size_t)row * DK + cv * 8);
      *reinterpret_cast<uint4*>(sKr + row * DK + cv * 8) = *reinterpret_cast<const uint4*>(kc + (size_t)row * DK + cv * 8);
      *reinterpret_cast<uint4*>(sGr + row * DK + cv * 8) = *reinterpret_cast<const uint4*>(gc + (size_t)row * DK + cv * 8);
    }
  }
  __syncthreads();
  for (int jt = 0; jt < rv; jt++) {
    const float x = bf2f(sGr[jt * DK + d]);
    const float la = GM == kGateLogit ? (fminf(x, 0.f) - log1pf(__expf(-fabsf(x)))) * inv_tau
                                      : fminf(x, 0.f);
    const float a = __expf(la);
    const float kd = bf2f(sKr[jt * DK + d]), qd = bf2f(sQr[jt * DK + d]);
    float op[CPT];
#pragma unroll
    for (int i = 0; i < CPT; i++) {
      s[i] = a * s[i] + kd * bf2f(sV[jt * Lds::LDV + p * CPT + i]);
      op[i] = qd * s[i];
    }
    // over the wave's key dimensions (lanes with equal p), then over the waves
#pragma unroll
    for (int i = 0; i < CPT; i++) {
#pragma unroll
      for (int off = TPD; off < 64; off <<= 1) op[i] += __shfl_xor(op[i], off, 64);
    }
    if (lane < TPD) {
#pragma unroll
      for (int i = 0; i < CPT; i++) sOp[wv * DV + p * CPT + i] = op[i];
    }
    __syncthreads();
    if (tid < DV) {
      float o = 0.f;
#pragma unroll
      for (int w8 = 0; w8 < NW; w8++) o += sOp[w8 * DV + tid];
      orow[(size_t)jt * DV + tid] = f2bf(o);
    }
    __syncthreads();
  }
  // state back to the accumulators
#pragma unroll
  for (int i = 0; i < CPT; i++) sSf[d * DV + p * CPT + i] = s[i];
  __syncthreads();
  if (is_state) W.load(sSf, DV, wv - 4, lane);
  __syncthreads();  // the region is reused by the state copy and later rows
}

// ------------------------------------------------ phase A: state maps
// grid (Q, units) with Q = (P-1) R: map i covers sub-segment i % R of output
// segment i / R, from a zero start: S^T Diag(E_C) + V^T Kh per chunk, and the
// product of the chunk decays.  All eight waves carry state tiles.
template <int DK, int DV, int GM>
__global__ void __launch_bounds__(NT, 2)
gla_bf16_state(const bf16_t* __restrict__ kk, const bf16_t* __restrict__ vv,
               const bf16_t* __restrict__ gg, float* __restrict__ ws_state,
               float* __restrict__ ws_dec, int T_len, int S, int R, int NQ, float inv_tau) {
  using Lds = GlaStateLds<DK, DV>;
  constexpr int SPT = DK / NW;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  auto bK = [&](int b) { return reinterpret_cast<bf16_t*>(smem + b * Lds::szBuf + Lds::oK); };
  auto bV = [&](int b) { return reinterpret_cast<bf16_t*>(smem + b * Lds::szBuf + Lds::oV); };
  auto bEc = [&](int b) { return reinterpret_cast<float*>(smem + b * Lds::szBuf + Lds::oEc); };

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int i = blockIdx.x, unit = blockIdx.y;
  const int d0 = wv * SPT;
  const int nchunks = (T_len + C - 1) / C;
  const int sa = (S + R - 1) / R;
  const int seg_end = min((i / R + 1) * S, nchunks);
  const int c_begin = (i / R) * S + (i % R) * sa;
  const int c_end = min(c_begin + sa, seg_end);
  float* dst = ws_state + ((size_t)unit * NQ + i) * DK * DV;
  float* ddst = ws_dec + ((size_t)unit * NQ + i) * DK + d0;

  GlaTiles<DK, DV, NW> W;
  W.zero();
  float dec[SPT];
#pragma unroll
  for (int s = 0; s < SPT; s++) dec[s] = 1.f;
  if (c_begin >= c_end) {  // empty sub-segment: the identity map
    W.store(dst, DV, wv, lane);
    if (lane == 0) store_f32_row<SPT>(ddst, dec);
    return;
  }
  const size_t ub = (size_t)unit * T_len;
  const bf16_t* kb = kk + ub * DK + d0;
  const bf16_t* gb = gg + ub * DK + d0;
  const bf16_t* vb = vv + ub * DV;

  GateRow<SPT> rk, rg;
  Tile<DV> pv;
  auto load_chunk = [&](int ch, int tid_, int lane_) {
    const int t0 = ch * C, rv = min(C, T_len - t0);
    const size_t row = (size_t)(t0 + min(lane_, rv - 1)) * DK;
    rk.load(kb + row);
    rg.load(gb + row);
    pv.load_branchy(vb + (size_t)t0 * DV, rv, tid_);
  };
  auto stage_chunk = [&](int ch, int b, bool count, int tid_, int lane_) {
    const int rv = min(C, T_len - ch * C);
    pv.store_branchy(bV(b), Lds::LDV, rv, tid_);
    map_factors<SPT, Lds::LDQ, GM>(rk, rg, rv, inv_tau, lane_, d0, bK(b), bEc(b), dec, count);
  };

  load_chunk(c_begin, tid, lane);
  stage_chunk(c_begin, 0, true, tid, lane);
  load_chunk(min(c_begin + 1, c_end - 1), tid, lane);
  __syncthreads();
  int b = 0;
  for (int ch = c_begin; ch < c_end; ch++) {
    int lane_i = lane, tid_i = tid;  // re-derived per chunk (see the output kernel)
    asm volatile("" : "+v"(lane_i), "+v"(tid_i));
    // next chunk into the other buffer (the last chunk's again at the end,
    // into a buffer nobody reads, not counted in the decay), the one after
    // into registers, this chunk's state update: independent until the barrier
    stage_chunk(min(ch + 1, c_end - 1), b ^ 1, ch + 1 < c_end, tid_i, lane_i);
    load_chunk(min(ch + 2, c_end - 1), tid_i, lane_i);
    W.template carry<false>(bV(b), Lds::LDV, bK(b), Lds::LDQ, bEc(b), wv, lane_i);
    __syncthreads();
    b ^= 1;
  }
  W.store(dst, DV, wv, lane);
  if (lane == 0) store_f32_row<SPT>(ddst, dec);
}

// ----------------------------------------------------- phase B: scan
// One thread per (unit, state element), serial over the Q maps; the start
// state of output segment p is written to slot p before map p R is applied.
// The loads of a batch of maps are issued before any of the batch's stores;
// every store goes to a slot at or below the last one read.
template <int DK, int DV>
__global__ void __launch_bounds__(256)
gla_bf16_scan(float* __restrict__ ws_state, const float* __restrict__ ws_dec, const float* __restrict__ s0,
              int units, int P, int R, int NQ) {
  constexpr int NE = DK * DV;
  constexpr int BATCH = 8;
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long long)units * NE) return;
  const int unit = (int)(gid / NE), e = (int)(gid % NE);
  const int c = e / DV;
  float W = s0 ? s0[(size_t)unit * NE + e] : 0.f;
  float* st = ws_state + (size_t)unit * NQ * NE + e;
  const float* dc = ws_dec + (size_t)unit * NQ * DK + c;
  const int Q = (P - 1) * R;
  for (int i0 = 0; i0 < Q; i0 += BATCH) {
    float x[BATCH], d[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; u++) {
      if (i0 + u < Q) {
        x[u] = st[(size_t)(i0 + u) * NE];
        d[u] = dc[(size_t)(i0 + u) * DK];
      }
    }
#pragma unroll
    for (int u = 0; u < BATCH; u++) {
      const int i = i0 + u;
      if (i < Q) {
        if (i % R == 0) st[(size_t)(i / R) * NE] = W;
        W = d[u] * W + x[u];
      }
    }
  }
  st[(size_t)(P - 1) * NE] = W;
}

// ------------------------------------------------------ phase C: outputs
// Per chunk c (factor set b = c & 1): the contractions of chunk c (pass waves)
// beside the state waves' share of chunk c+1's factors and their carry; a
// barrier; the state copy, chunk c+1's v into the V slot and chunk c+2's q, k,
// g rows (loaded one chunk earlier as coalesced tiles) into set b; the loads
// of chunks c+3 and c+2; the pass waves' share of chunk c+1's factors (from
// set b^1); a barrier that also combines the exact-path votes.
template <int DK, int DV, int GM>
__global__ void __launch_bounds__(NT, 1)
gla_bf16_out(const bf16_t* __restrict__ qq, const bf16_t* __restrict__ kk,
             const bf16_t* __restrict__ vv, const bf16_t* __restrict__ gg,
             const float* __restrict__ s0, const float* __restrict__ ws_state,
             bf16_t* __restrict__ oo, float* __restrict__ sf, const float* __restrict__ ws_dec,
             int T_len, int S, int P, int NQ, int R, int fold, float inv_tau) {
  using Lds = GlaOutLds<DK, DV>;
  using ST = GlaTiles<DK, DV, 4>;
  constexpr int SPT = DK / NW;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  bf16_t* sV = reinterpret_cast<bf16_t*>(smem + Lds::oV);
  auto fQ = [&](int b) { return reinterpret_cast<bf16_t*>(smem + Lds::oF(b) + Lds::fQ); };
  auto fK = [&](int b) { return reinterpret_cast<bf16_t*>(smem + Lds::oF(b) + Lds::fK); };
  auto fEc = [&](int b) { return reinterpret_cast<float*>(smem + Lds::oEc + b * DK * 4); };
  bf16_t* sS = reinterpret_cast<bf16_t*>(smem + Lds::oS);
  auto fG = [&](int b) { return reinterpret_cast<bf16_t*>(smem + Lds::oG(b)); };
  int* sFlag = reinterpret_cast<int*>(smem + Lds::oFlag);

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const bool is_state = wv >= 4;
  const int sw = wv - 4;
  const int d0 = wv * SPT;  // this wave's key dimensions in the factor step
  const int seg = blockIdx.x, unit = blockIdx.y;
  const int nchunks = (T_len + C - 1) / C;
  const int c_begin = seg * S, c_end = min(c_begin + S, nchunks);
  const size_t ub = (size_t)unit * T_len;
  const bf16_t* qb = qq + ub * DK;
  const bf16_t* kb = kk + ub * DK;
  const bf16_t* gb = gg + ub * DK;
  const bf16_t* vb = vv + ub * DV;
  bf16_t* ob = oo + ub * DV;
  auto rows_of = [&](int ch) { return min(C, T_len - ch * C); };
  auto clamp = [&](int ch) { return min(ch, c_end - 1); };

  // raw tiles of later chunks in registers (coalesced loads): q, k, g three
  // chunks ahead (staged two ahead, into the factor set of their chunk), v two
  // ahead (staged one ahead, into the single V slot)
  Tile<DK> pq, pk, pg;
  Tile<DV> pv;
  auto load_qkg = [&](int ch, int tid_) {
    const int t0 = ch * C, rv = rows_of(ch);
    pq.load(qb + (size_t)t0 * DK, rv, tid_);
    pk.load(kb + (size_t)t0 * DK, rv, tid_);
    pg.load(gb + (size_t)t0 * DK, rv, tid_);
  };
  auto load_v = [&](int ch, int tid_) { pv.load(vb + (size_t)ch * C * DV, rows_of(ch), tid_); };
  auto stage_qkg = [&](int ch, int b, int tid_) {  // rows >= rv are zeroed
    const int rv = rows_of(ch);
    pq.store(fQ(b), Lds::LDQ, rv, tid_);
    pk.store(fK(b), Lds::LDQ, rv, tid_);
    pg.store(fG(b), Lds::LDQ, rv, tid_);
  };
  auto stage_v = [&](int ch, int tid_) { pv.store(sV, Lds::LDV, rows_of(ch), tid_); };
  auto factors = [&](int ch, int b, int lane_) -> bool {
    return out_factors<SPT, Lds::LDQ, GM>(fQ(b), fK(b), fG(b), rows_of(ch), inv_tau, lane_, d0, fEc(b));
  };

  ST W;
  bool slow;
  load_qkg(c_begin, tid);
  load_v(c_begin, tid);
  if (is_state) {
    if (P > 1 && !fold) {
      W.load(ws_state + ((size_t)unit * NQ + seg) * DK * DV, DV, sw, lane);  // from the scan
    } else {
      W.load(s0 ? s0 + (size_t)unit * DK * DV : nullptr, DV, sw, lane);
      // the start state as the segment recurrence over the sub-segment maps
      // before this segment (one map at a time: the chunk's tiles are live)
      const int nm = seg * R;
      const float* mp = ws_state + (size_t)unit * NQ * DK * DV;
      const float* dp = ws_dec + (size_t)unit * NQ * DK;
      for (int p = 0; p < nm; p++) {
        typename ST::MapRegs x;
        W.load_map(x, mp + (size_t)p * DK * DV, sw, lane);
        W.fold(x, dp + (size_t)p * DK, sw, lane);
      }
    }
    W.store_copy(sS, Lds::LDS, sw, lane);
  }
  stage_qkg(c_begin, 0, tid);
  stage_v(c_begin, tid);
  load_qkg(clamp(c_begin + 1), tid);
  load_v(clamp(c_begin + 1), tid);
  __syncthreads();
  slow = block_any(factors(c_begin, 0, lane), sFlag, 0, lane, wv);
  stage_qkg(clamp(c_begin + 1), 1, tid);
  load_qkg(clamp(c_begin + 2), tid);
  __syncthreads();

  int b = 0;  // factor set of the current chunk
  for (int ch = c_begin; ch < c_end; ch++) {
    // lane / thread indices re-derived each chunk: keeps the compiler from
    // holding every per-lane LDS address of the loop in registers across it
    int lane_i = lane, tid_i = tid;
    asm volatile("" : "+v"(lane_i), "+v"(tid_i));
    const int t0 = ch * C, rv = rows_of(ch);
    bool small = false;
    if (!slow) {
      if (!is_state) {
        bf16_t* orow = ob + (size_t)t0 * DV;
        // pass waves hold no state: dropping it frees these registers for the passes
        W.zero();
        switch (wv) {
          case 0: gla_pass_chunk<DK, DV, 0>(lane_i, fQ(b), fK(b), sV, sS, orow, rv); break;
          case 1: gla_pass_chunk<DK, DV, 1>(lane_i, fQ(b), fK(b), sV, sS, orow, rv); break;
          case 2: gla_pass_chunk<DK, DV, 2>(lane_i, fQ(b), fK(b), sV, sS, orow, rv); break;
          default: gla_pass_chunk<DK, DV, 3>(lane_i, fQ(b), fK(b), sV, sS, orow, rv); break;
        }
      } else {
        // the state waves take the next chunk's factors first: their gate
        // arithmetic then overlaps the pass waves' contractions on each SIMD
        small = factors(clamp(ch + 1), b ^ 1, lane_i);
        W.template carry<true>(sV, Lds::LDV, fK(b), Lds::LDQ, fEc(b), sw, lane_i);
      }
    } else {
      gla_exact_chunk<DK, DV, GM>(W, rv, smem + Lds::oX(b), sV, qb + (size_t)t0 * DK,
                              kb + (size_t)t0 * DK, gb + (size_t)t0 * DK, ob + (size_t)t0 * DV, tid_i,
                              inv_tau);
    }
    // every wave is done with the copy of S, the V slot and this chunk's set
    __syncthreads();
    if (is_state) W.store_copy(sS, Lds::LDS, sw, lane_i);
    // the next chunk's v into the V slot, chunk ch+2's rows into this chunk's
    // set, then the loads of chunks ch+3 (q, k, g) and ch+2 (v) (unconditional,
    // clamped: no branch blurs the load-count waits)
    stage_v(clamp(ch + 1), tid_i);
    stage_qkg(clamp(ch + 2), b, tid_i);
    load_qkg(clamp(ch + 3), tid_i);
    load_v(clamp(ch + 2), tid_i);
    // the next chunk's factors (this one again at the end, into a set nobody
    // reads) by the waves that have not computed them yet: the pass waves'
    // gate arithmetic runs here, beside the state waves' copy of S (the rows
    // it reads, set b^1 and its g tile, are not written in this chunk)
    if (slow || !is_state) small = factors(clamp(ch + 1), b ^ 1, lane_i);
    slow = block_any(small, sFlag, ch - c_begin + 1, lane_i, wv);
    b ^= 1;
  }

  if (seg == P - 1 && is_state && sf) W.store(sf + (size_t)unit * DK * DV, DV, sw, lane);
}

// ------------------------------------------------------------ launcher
template <int DK, int DV, int GM>
static int launch_gla(const GlaLaunch& a) {
  using LO = GlaOutLds<DK, DV>;
  using LS = GlaStateLds<DK, DV>;
  const int units = a.B * a.H;
  const int nchunks = (a.T + C - 1) / C;
  const int S = a.chunks_per_seg;
  const int P = (nchunks + S - 1) / S;
  const int R = P > 1 ? a.state_split : 1;
  const int Q = (P - 1) * R;
  const int NQ = Q > P ? Q : P;
  const float inv_tau = 1.0f / a.tau;
  hipStream_t st = (hipStream_t)a.stream;
  static const bool lds_set = [] {  // once per instantiation and process
    (void)hipFuncSetAttribute((const void*)gla_bf16_out<DK, DV, GM>, hipFuncAttributeMaxDynamicSharedMemorySize,
                        LO::total);
    (void)hipFuncSetAttribute((const void*)gla_bf16_state<DK, DV, GM>, hipFuncAttributeMaxDynamicSharedMemorySize,
                        LS::total);
    return true;
  }();
  (void)lds_set;
  // As in the GSA forward: with at most kMaxFoldedMaps maps before the last
  // segment, the output workgroups fold them into their start states (no scan
  // launch), unless the final state is written over s0.
  const int fold = P > 1 && Q <= kMaxFoldedMaps && !(a.sf && a.sf == a.s0);
  if (P > 1) {
    launch_timed(gla_bf16_state<DK, DV, GM>, dim3(Q, units), dim3(NT), LS::total, a.stream, a.events, 0, 1,
                 (const bf16_t*)a.k, (const bf16_t*)a.v, (const bf16_t*)a.g, a.ws_state, a.ws_dec, a.T,
                 S, R, NQ, inv_tau);
    if (!fold) {
      const long long ne = (long long)units * DK * DV;
      hipLaunchKernelGGL((gla_bf16_scan<DK, DV>), dim3((unsigned)((ne + 255) / 256)), dim3(256), 0, st,
                         a.ws_state, (const float*)a.ws_dec, a.s0, units, P, R, NQ);
    }
  } else {
    record_event(a.events, 0, a.stream);
    record_event(a.events, 1, a.stream);
  }
  launch_timed(gla_bf16_out<DK, DV, GM>, dim3(P, units), dim3(NT), LO::total, a.stream, a.events, 2, 3,
               (const bf16_t*)a.q, (const bf16_t*)a.k, (const bf16_t*)a.v, (const bf16_t*)a.g, a.s0,
               (const float*)a.ws_state, (bf16_t*)a.o, a.sf, (const float*)a.ws_dec, a.T, S, P, NQ, R,
               fold, inv_tau);
  return 0;
}

}  // namespace bfk

#define GLA_BF16_CASE(DKC, DVC)                                      \
  if (dk == DKC && dv == DVC) {                                      \
    static_assert(bfk::GlaOutLds<DKC, DVC>::total <= kLdsBytes, "LDS"); \
    if (query) return bfk::GlaOutLds<DKC, DVC>::total;               \
    return a->gate_mode == kGateLogit ? bfk::launch_gla<DKC, DVC, kGateLogit>(*a)           \
                                      : bfk::launch_gla<DKC, DVC, kGateLogDecay>(*a);       \
  }

// Returns: query -> LDS bytes (>0) or -1 if unsupported; launch -> 0 or -1.
int gla_dispatch_bf16(int dk, int dv, const GlaLaunch* a, bool query) {
  GLA_BF16_CASE(128, 128)
  GLA_BF16_CASE(64, 64)
  return -1;
}

}  // namespace gsa
