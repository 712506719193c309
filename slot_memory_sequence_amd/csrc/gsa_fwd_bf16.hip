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
// the outputs (gsa_bf16_out).  A chunk whose decay product falls below e^-40
// in some slot is run as the exact token recurrence instead (no division by a
// decay product).
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"

namespace gsa {
namespace bfk {

constexpr int C = 64;   // chunk length
constexpr int NW = 8;   // waves per workgroup
constexpr int NT = NW * 64;
constexpr float kFastMinLogDecay = -40.f;  // log of the smallest whole-chunk decay the factors allow

typedef __attribute__((ext_vector_type(8))) float f32x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4v;

__device__ __forceinline__ f32x4 mma(const bf16x8& a, const bf16x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// two accumulator quads -> one operand fragment (round to nearest even)
__device__ __forceinline__ bf16x8 pack8(const f32x4& a, const f32x4& b) {
  f32x8 x = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_convertvector(x, bf16x8);
}
__device__ __forceinline__ bf16x4v pack4(const f32x4& a) { return __builtin_convertvector(a, bf16x4v); }

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Row-major [row][k] tile: lane l gets 8 consecutive k at row row0 + l%16,
// column k0 + 8*(l/16)  (MFMA operand order, standard k).
__device__ __forceinline__ bf16x8 ld_row(const bf16_t* base, int ld, int row0, int k0, int lane) {
  return *reinterpret_cast<const bf16x8*>(base + (row0 + (lane & 15)) * ld + k0 + 8 * (lane >> 4));
}

// Row-major [row][k] tile, permuted k: lane l gets 4 consecutive k from klo and
// 4 from khi (both already include the lane group's offset) at row row0 + l%16.
__device__ __forceinline__ bf16x8 ld_row2(const bf16_t* base, int ld, int row0, int klo, int khi,
                                          int lane) {
  const bf16_t* p = base + (row0 + (lane & 15)) * ld;
  bf16x4v lo = *reinterpret_cast<const bf16x4v*>(p + klo);
  bf16x4v hi = *reinterpret_cast<const bf16x4v*>(p + khi);
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Row-major [k][n] tile read column-wise with the LDS transpose read: lane l
// gets tile[klo + jj][n0 + l%16] and tile[khi + jj][n0 + l%16], jj = 0..3,
// where klo / khi already include the lane group's offset.
__device__ __forceinline__ bf16x8 ld_col(const bf16_t* base, int ld, int n0, int klo, int khi,
                                         int lane) {
  const int L = lane & 15;
  const bf16_t* p0 = base + (klo + (L >> 2)) * ld + n0 + 4 * (L & 3);
  const bf16_t* p1 = base + (khi + (L >> 2)) * ld + n0 + 4 * (L & 3);
  bf16x4_raw lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((GSA_LDS bf16x4_raw*)(p0));
  bf16x4_raw hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((GSA_LDS bf16x4_raw*)(p1));
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

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
  // fast path
  static constexpr int oW = oR;                        // bf16 copy of W [M][DK+DV]
  static constexpr int oX = oW + M * LDW * 2;          // X [C][M] bf16
  static constexpr int oZ = oX + C * LDX * 2;          // Z [C][M] bf16
  static constexpr int oE = oZ + C * LDX * 2;          // E [C][M] fp32
  static constexpr int szFast = oE + C * LDE * 4 - oR;
  // exact-recurrence path
  static constexpr int oWf = oR;                       // fp32 W [M][DK+DV]
  static constexpr int oLa = oWf + M * (DK + DV) * 4;  // log alpha [C][M] fp32
  static constexpr int oZs = oLa + C * M * 4;          // slot scores [M] fp32
  static constexpr int oOp = oZs + M * 4;              // output partials [NW][DV] fp32
  static constexpr int szSlow = oOp + NW * DV * 4 - oR;
  static constexpr int oDec = oR + (szFast > szSlow ? szFast : szSlow);  // [M] fp32
  static constexpr int total = oDec + M * 4;
  static_assert(oK % 16 == 0 && oV % 16 == 0 && oW % 16 == 0 && oX % 16 == 0 && oZ % 16 == 0 &&
                    oE % 16 == 0 && oLa % 16 == 0 && oOp % 16 == 0 && oDec % 16 == 0,
                "LDS tiles must stay 16-byte aligned");
};

template <int DK, int DV, int M>
struct StateLds {
  static constexpr int PAD = 8;
  static constexpr int LDQ = DK + PAD, LDV = DV + PAD, LDX = M + PAD;
  static constexpr int oK = 0;
  static constexpr int oV = oK + C * LDQ * 2;
  static constexpr int oZ = oV + C * LDV * 2;
  static constexpr int oDec = oZ + C * LDX * 2;
  static constexpr int total = oDec + M * 4;
};

// ------------------------------------------------------- global tile I/O
// [C][D] bf16 chunk tile moved as 16-byte vectors by the 512 threads.
template <int D>
struct Tile {
  static constexpr int VPR = D / 8;
  static constexpr int NV = C * VPR / NT;
  static_assert(NV >= 1 && (C * VPR) % NT == 0, "tile/thread mismatch");
  uint4 r[NV];
  // rows >= rows_valid (>= 1) read the last valid row and are then zeroed, so
  // the loads need no branches
  __device__ __forceinline__ void load(const bf16_t* __restrict__ base, int rows_valid, int tid) {
#pragma unroll
    for (int i = 0; i < NV; i++) {
      const int idx = tid + NT * i, row = idx / VPR, cv = idx % VPR;
      const int rr = min(row, rows_valid - 1);
      const uint4 x = *reinterpret_cast<const uint4*>(base + rr * D + cv * 8);
      const bool ok = row < rows_valid;
      r[i] = make_uint4(ok ? x.x : 0u, ok ? x.y : 0u, ok ? x.z : 0u, ok ? x.w : 0u);
    }
  }
  __device__ __forceinline__ void store(bf16_t* dst, int ld, int tid) const {
#pragma unroll
    for (int i = 0; i < NV; i++) {
      const int idx = tid + NT * i, row = idx / VPR, cv = idx % VPR;
      *reinterpret_cast<uint4*>(dst + row * ld + cv * 8) = r[i];
    }
  }
};

// SPT gate logits of one token row (SPT = 4 or 8 bf16 = 8 or 16 bytes).
template <int SPT>
struct GateRow {
  static_assert(SPT == 4 || SPT == 8, "gate row width");
  typedef typename std::conditional<SPT == 8, uint4, uint2>::type V;
  V r;
  // p must point at a readable row even when !valid (the caller clamps it)
  __device__ __forceinline__ void load(const bf16_t* __restrict__ p, bool valid) {
    const V x = *reinterpret_cast<const V*>(p);
    r = valid ? x : V{};
  }
  __device__ __forceinline__ float at(int s) const { return bf2f(reinterpret_cast<const bf16_t*>(&r)[s]); }
};

// Gates of SPT slots for token row = lane of a chunk, for the output pass:
// w = 1 - alpha and G = chunk-local inclusive cumulative sum of log alpha (one
// wave scan).  E_j = exp(G_j); the decay from token r to the chunk end is
// exp(G_C - G_r).  Rows past the end of the sequence are identity steps
// (log alpha = 0, write 0).  Only chunks with G_C >= -40 in every slot use
// these factors, so every exponential below stays finite there.
template <int SPT>
struct LogGates {
  float w[SPT], G[SPT];
  __device__ __forceinline__ void compute(const GateRow<SPT>& g, bool valid, float inv_tau, int lane) {
#pragma unroll
    for (int s = 0; s < SPT; s++) {
      const float x = g.at(s);
      const float la = (fminf(x, 0.f) - log1pf(__expf(-fabsf(x)))) * inv_tau;
      G[s] = valid ? la : 0.f;
      w[s] = valid ? -expm1f(la) : 0.f;
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
#pragma unroll
      for (int s = 0; s < SPT; s++) {
        const float up = __shfl_up(G[s], off, 64);
        if (lane >= off) G[s] += up;
      }
    }
  }
};

// Gates for the state-map pass: w = 1 - alpha and the exclusive suffix product
// S_r = prod_{i>r} alpha_i (one wave scan, exact also for alpha = 0), plus the
// whole-chunk product.
template <int SPT>
struct SuffixGates {
  float w[SPT], S[SPT], dec[SPT];
  __device__ __forceinline__ void compute(const GateRow<SPT>& g, bool valid, float inv_tau, int lane) {
    float a[SPT];
#pragma unroll
    for (int s = 0; s < SPT; s++) {
      float av, wv;
      gate_alpha_w(g.at(s), inv_tau, av, wv);
      a[s] = valid ? av : 1.f;
      w[s] = valid ? wv : 0.f;
      S[s] = a[s];
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
#pragma unroll
      for (int s = 0; s < SPT; s++) {
        const float dn = __shfl_down(S[s], off, 64);
        if (lane + off < 64) S[s] *= dn;
      }
    }
    // S is now the inclusive suffix product; lane 0 holds the whole product
#pragma unroll
    for (int s = 0; s < SPT; s++) {
      dec[s] = __shfl(S[s], 0, 64);
      const float nx = __shfl_down(S[s], 1, 64);
      S[s] = (lane == 63) ? 1.f : nx;
    }
  }
};

// SPT consecutive floats -> SPT bf16 stored as one 8- or 16-byte vector
template <int SPT>
__device__ __forceinline__ void store_bf16_row(bf16_t* dst, const float* v) {
  if constexpr (SPT == 8) {
    f32x8 x = {v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7]};
    *reinterpret_cast<bf16x8*>(dst) = __builtin_convertvector(x, bf16x8);
  } else {
    f32x4 x = {v[0], v[1], v[2], v[3]};
    *reinterpret_cast<bf16x4v*>(dst) = __builtin_convertvector(x, bf16x4v);
  }
}
template <int SPT>
__device__ __forceinline__ void store_f32_row(float* dst, const float* v) {
#pragma unroll
  for (int s = 0; s < SPT; s += 4)
    *reinterpret_cast<float4*>(dst + s) = make_float4(v[s], v[s + 1], v[s + 2], v[s + 3]);
}

// ------------------------------------------------------------ state tiles
// W^T held in MFMA accumulators by NSW waves: wave sw owns column tiles
// [sw*NCW, (sw+1)*NCW) of W (columns 0..DK-1 are Kt, DK.. are Vt) and all M
// slots.  Lane l of tile (n, ct) holds W[16ct + l%16][16(sw*NCW+n) + 4(l/16) + i].
template <int DK, int DV, int M, int NSW>
struct StateTiles {
  static constexpr int MT = M / 16;
  static constexpr int NCT = (DK + DV) / 16;
  static constexpr int NCW = NCT / NSW;
  static_assert(NCT % NSW == 0 && NCW >= 1, "state columns must split evenly");
  static_assert((DK / 16) % NCW == 0, "a wave's columns must lie in one of Kt / Vt");
  f32x4 st[NCW][MT];

  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int n = 0; n < NCW; n++)
#pragma unroll
      for (int ct = 0; ct < MT; ct++) st[n][ct] = zero4();
  }
  __device__ __forceinline__ int col(int sw, int n, int lane) const {
    return 16 * (sw * NCW + n) + 4 * (lane >> 4);
  }
  // src [M][DK+DV] fp32 (one map/state of the workspace)
  __device__ __forceinline__ void load_w(const float* __restrict__ src, int sw, int lane) {
#pragma unroll
    for (int n = 0; n < NCW; n++)
#pragma unroll
      for (int ct = 0; ct < MT; ct++) {
        const float4 x = *reinterpret_cast<const float4*>(
            src + (size_t)(16 * ct + (lane & 15)) * (DK + DV) + col(sw, n, lane));
        st[n][ct] = f32x4{x.x, x.y, x.z, x.w};
      }
  }
  // k0 [M][DK], v0 [M][DV], each nullable (zeros)
  __device__ __forceinline__ void load_kv(const float* __restrict__ k0, const float* __restrict__ v0,
                                          int sw, int lane) {
#pragma unroll
    for (int n = 0; n < NCW; n++) {
      const int cl = col(sw, n, lane);
#pragma unroll
      for (int ct = 0; ct < MT; ct++) {
        const int c = 16 * ct + (lane & 15);
        const float* p = cl < DK ? (k0 ? k0 + (size_t)c * DK + cl : nullptr)
                                 : (v0 ? v0 + (size_t)c * DV + cl - DK : nullptr);
        if (p) {
          const float4 x = *reinterpret_cast<const float4*>(p);
          st[n][ct] = f32x4{x.x, x.y, x.z, x.w};
        } else {
          st[n][ct] = zero4();
        }
      }
    }
  }
  __device__ __forceinline__ void store_w(float* __restrict__ dst, int sw, int lane) const {
#pragma unroll
    for (int n = 0; n < NCW; n++)
#pragma unroll
      for (int ct = 0; ct < MT; ct++)
        *reinterpret_cast<float4*>(dst + (size_t)(16 * ct + (lane & 15)) * (DK + DV) + col(sw, n, lane)) =
            make_float4(st[n][ct][0], st[n][ct][1], st[n][ct][2], st[n][ct][3]);
  }
  __device__ __forceinline__ void store_kv(float* __restrict__ kf, float* __restrict__ vf, int sw,
                                           int lane) const {
#pragma unroll
    for (int n = 0; n < NCW; n++) {
      const int cl = col(sw, n, lane);
#pragma unroll
      for (int ct = 0; ct < MT; ct++) {
        const int c = 16 * ct + (lane & 15);
        float* p = cl < DK ? (kf ? kf + (size_t)c * DK + cl : nullptr)
                           : (vf ? vf + (size_t)c * DV + cl - DK : nullptr);
        if (p) *reinterpret_cast<float4*>(p) = make_float4(st[n][ct][0], st[n][ct][1], st[n][ct][2], st[n][ct][3]);
      }
    }
  }
  // bf16 copy of W, row-major [M][ldw]
  __device__ __forceinline__ void store_copy(bf16_t* sW, int ldw, int sw, int lane) const {
#pragma unroll
    for (int n = 0; n < NCW; n++)
#pragma unroll
      for (int ct = 0; ct < MT; ct++)
        *reinterpret_cast<bf16x4v*>(sW + (16 * ct + (lane & 15)) * ldw + col(sw, n, lane)) = pack4(st[n][ct]);
  }
  // one chunk: W^T <- W^T Diag(E_C) + [K|V]^T Z
  __device__ __forceinline__ void carry(const bf16_t* sK, int ldk, const bf16_t* sV, int ldv,
                                        const bf16_t* sZ, int ldz, const float* sDec, int sw,
                                        int lane) {
    const int L = lane & 15, g = lane >> 4;
#pragma unroll
    for (int ct = 0; ct < MT; ct++) {
      const float d = sDec[16 * ct + L];
#pragma unroll
      for (int n = 0; n < NCW; n++)
#pragma unroll
        for (int i = 0; i < 4; i++) st[n][ct][i] *= d;
    }
#pragma unroll
    for (int r0 = 0; r0 < C; r0 += 32) {
      bf16x8 zb[MT];
#pragma unroll
      for (int ct = 0; ct < MT; ct++) zb[ct] = ld_col(sZ, ldz, 16 * ct, r0 + 8 * g, r0 + 8 * g + 4, lane);
#pragma unroll
      for (int n = 0; n < NCW; n++) {
        const int c0 = 16 * (sw * NCW + n);
        const bf16x8 a = c0 < DK ? ld_col(sK, ldk, c0, r0 + 8 * g, r0 + 8 * g + 4, lane)
                                 : ld_col(sV, ldv, c0 - DK, r0 + 8 * g, r0 + 8 * g + 4, lane);
#pragma unroll
        for (int ct = 0; ct < MT; ct++) st[n][ct] = mma(a, zb[ct], st[n][ct]);
      }
    }
  }
};

// -------------------------------------------------------- pass-wave chunk
// Token rows 16J..16J+15 of the chunk: both passes, the slot softmax and the
// output rows.  Reads sQ, sK, sV, sX, sE and the bf16 state copy sW.
template <int DK, int DV, int M>
__device__ __forceinline__ void pass_chunk(int J, int lane, const bf16_t* sQ, const bf16_t* sK,
                                           const bf16_t* sV, const bf16_t* sW, const bf16_t* sX,
                                           const float* sE, bf16_t* __restrict__ orow, int rv) {
  using Lds = OutLds<DK, DV, M>;
  constexpr int MT = M / 16, KQ = DK / 32, NP = M / 32, NVT = DV / 16;
  const int L = lane & 15, g = lane >> 4;
  const int j = 16 * J + L;  // this lane's token column

  // Q^T operand: B[d][j] = Q[j][d]
  bf16x8 qf[KQ];
#pragma unroll
  for (int s = 0; s < KQ; s++) qf[s] = ld_row(sQ, Lds::LDQ, 16 * J, 32 * s, lane);

  // A^T[r][j] = k_r . q_j for row tiles R <= J, causal mask on the diagonal tile
  f32x4 at[4];
#pragma unroll
  for (int R = 0; R < 4; R++) {
    at[R] = zero4();
    if (R <= J) {
#pragma unroll
      for (int s = 0; s < KQ; s++) at[R] = mma(ld_row(sK, Lds::LDQ, 16 * R, 32 * s, lane), qf[s], at[R]);
      if (R == J) {
#pragma unroll
        for (int i = 0; i < 4; i++)
          if (4 * g + i > L) at[R][i] = 0.f;
      }
    }
  }
  const bf16x8 af0 = pack8(at[0], at[1]);
  const bf16x8 af1 = pack8(at[2], at[3]);
  const bool two = J >= 2;  // second r-pair needed

  // pass 1: o'^T[c][j] = E[j][c] (Wk[c].q_j + sum_r X[r][c] A^T[r][j])
  f32x4 op[MT];
  f32x4 ev[MT];
#pragma unroll
  for (int ct = 0; ct < MT; ct++) {
    f32x4 acc = zero4();
#pragma unroll
    for (int s = 0; s < KQ; s++) acc = mma(ld_row(sW, Lds::LDW, 16 * ct, 32 * s, lane), qf[s], acc);
    acc = mma(ld_col(sX, Lds::LDX, 16 * ct, 4 * g, 16 + 4 * g, lane), af0, acc);
    if (two) acc = mma(ld_col(sX, Lds::LDX, 16 * ct, 32 + 4 * g, 48 + 4 * g, lane), af1, acc);
    const float4 e = *reinterpret_cast<const float4*>(sE + j * Lds::LDE + 16 * ct + 4 * g);
    ev[ct] = f32x4{e.x, e.y, e.z, e.w};
#pragma unroll
    for (int i = 0; i < 4; i++) op[ct][i] = acc[i] * ev[ct][i];
  }

  // slot softmax of token j: over (ct, i) in-lane and the four lane groups
  float mx = op[0][0];
#pragma unroll
  for (int ct = 0; ct < MT; ct++)
#pragma unroll
    for (int i = 0; i < 4; i++) mx = fmaxf(mx, op[ct][i]);
  mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  float sm = 0.f;
#pragma unroll
  for (int ct = 0; ct < MT; ct++)
#pragma unroll
    for (int i = 0; i < 4; i++) {
      op[ct][i] = __expf(op[ct][i] - mx);
      sm += op[ct][i];
    }
  sm += __shfl_xor(sm, 16, 64);
  sm += __shfl_xor(sm, 32, 64);
  const float inv = 1.f / sm;
  // (s*E)^T as B operands over slot pairs (permuted slot index)
  bf16x8 sb[NP];
#pragma unroll
  for (int p = 0; p < NP; p++) {
    f32x4 a, b;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      a[i] = op[2 * p][i] * inv * ev[2 * p][i];
      b[i] = op[2 * p + 1][i] * inv * ev[2 * p + 1][i];
    }
    sb[p] = pack8(a, b);
  }

  // pass 2 scores: A2^T[r][j] = sum_c X[r][c] (s*E)[j][c], r tiles R <= J
  f32x4 a2[4];
#pragma unroll
  for (int R = 0; R < 4; R++) {
    a2[R] = zero4();
    if (R <= J) {
#pragma unroll
      for (int p = 0; p < NP; p++)
        a2[R] = mma(ld_row2(sX, Lds::LDX, 16 * R, 32 * p + 4 * g, 32 * p + 16 + 4 * g, lane), sb[p], a2[R]);
      if (R == J) {
#pragma unroll
        for (int i = 0; i < 4; i++)
          if (4 * g + i > L) a2[R][i] = 0.f;
      }
    }
  }
  const bf16x8 a2f0 = pack8(a2[0], a2[1]);
  const bf16x8 a2f1 = pack8(a2[2], a2[3]);

  // o^T[n][j] = sum_c Wv[c][n] (s*E)[j][c] + sum_r V[r][n] A2^T[r][j]
  const bool store = j < rv;
#pragma unroll
  for (int nt = 0; nt < NVT; nt++) {
    f32x4 acc = zero4();
#pragma unroll
    for (int p = 0; p < NP; p++)
      acc = mma(ld_col(sW + DK, Lds::LDW, 16 * nt, 32 * p + 4 * g, 32 * p + 16 + 4 * g, lane), sb[p], acc);
    acc = mma(ld_col(sV, Lds::LDV, 16 * nt, 4 * g, 16 + 4 * g, lane), a2f0, acc);
    if (two) acc = mma(ld_col(sV, Lds::LDV, 16 * nt, 32 + 4 * g, 48 + 4 * g, lane), a2f1, acc);
    if (store) *reinterpret_cast<bf16x4v*>(orow + (size_t)j * DV + 16 * nt + 4 * g) = pack4(acc);
  }
}

// ------------------------------------------------ exact chunk recurrence
// Runs one chunk token by token: Kt, Vt <- Diag(alpha) (.) + (1-alpha)[k|v]^T,
// s = softmax over slots of Kt q, o = Vt^T s (Sec. 3.2 recurrent form).  Used
// for chunks whose decay product is too small for the factorised chunk form.
// The state waves' accumulators W are written to LDS, advanced there by all
// threads, and read back.  Contains workgroup barriers: all threads call it.
template <int DK, int DV, int M>
__device__ __forceinline__ void exact_chunk(StateTiles<DK, DV, M, 4>& W, const GateRow<M / NW>& pg,
                                            int rv, float inv_tau, unsigned char* smem,
                                            const bf16_t* sQ, const bf16_t* sK, const bf16_t* sV,
                                            bf16_t* __restrict__ orow, int tid) {
  using Lds = OutLds<DK, DV, M>;
  constexpr int SPT = M / NW;
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

  // state and log-gates to LDS (the region held the fast path's factors and
  // the bf16 state copy; all of their readers passed the last barrier)
  if (is_state) W.store_w(sWf, sw, lane);
#pragma unroll
  for (int s = 0; s < SPT; s++) {
    const float x = pg.at(s);
    const float la = (fminf(x, 0.f) - log1pf(__expf(-fabsf(x)))) * inv_tau;
    sLa[lane * M + wv * SPT + s] = lane < rv ? la : 0.f;
  }
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
    // slot softmax, computed by every wave; lane l < M holds slot l
    const float zl = lane < M ? sZs[lane] : -INFINITY;
    float mx = zl;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    const float el = lane < M ? __expf(zl - mx) : 0.f;
    const float sm = sum64(el);
    const float sc = __shfl(el, c, 64) / sm;
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
      orow[(size_t)jt * DV + tid] = f2bf(o);
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
}

// ------------------------------------------------ phase A: segment maps
// grid (P-1, units).  Map of segment seg from a zero start:
// D = sum over its tokens of Diag(prod_{i>r} alpha_i)(1-alpha_r)[k_r|v_r]^T and
// the segment decay product.  All eight waves carry state columns.
template <int DK, int DV, int M>
__global__ void __launch_bounds__(NT, 1)
gsa_bf16_state(const bf16_t* __restrict__ kk, const bf16_t* __restrict__ vv,
               const bf16_t* __restrict__ gg, float* __restrict__ ws_state,
               float* __restrict__ ws_dec, int T_len, int S, int P, float inv_tau) {
  using Lds = StateLds<DK, DV, M>;
  constexpr int SPT = M / NW;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  bf16_t* sK = reinterpret_cast<bf16_t*>(smem + Lds::oK);
  bf16_t* sV = reinterpret_cast<bf16_t*>(smem + Lds::oV);
  bf16_t* sZ = reinterpret_cast<bf16_t*>(smem + Lds::oZ);
  float* sDec = reinterpret_cast<float*>(smem + Lds::oDec);

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int seg = blockIdx.x, unit = blockIdx.y;
  const int nchunks = (T_len + C - 1) / C;
  const int c_begin = seg * S, c_end = min(c_begin + S, nchunks);
  const bf16_t* kb = kk + (size_t)unit * T_len * DK;
  const bf16_t* vb = vv + (size_t)unit * T_len * DV;
  const bf16_t* gb = gg + (size_t)unit * T_len * M + wv * SPT;

  StateTiles<DK, DV, M, NW> W;
  W.zero();
  float segdec[SPT];
#pragma unroll
  for (int s = 0; s < SPT; s++) segdec[s] = 1.f;

  Tile<DK> pk;
  Tile<DV> pv;
  GateRow<SPT> pg;
  {
    const int t0 = c_begin * C, rv = min(C, T_len - t0);
    pk.load(kb + (size_t)t0 * DK, rv, tid);
    pv.load(vb + (size_t)t0 * DV, rv, tid);
    pg.load(gb + (size_t)(t0 + min(lane, rv - 1)) * M, lane < rv);
  }
  for (int ch = c_begin; ch < c_end; ch++) {
    const int t0 = ch * C, rv = min(C, T_len - t0);
    pk.store(sK, Lds::LDQ, tid);
    pv.store(sV, Lds::LDV, tid);
    SuffixGates<SPT> gt;
    gt.compute(pg, lane < rv, inv_tau, lane);
    float z[SPT];
#pragma unroll
    for (int s = 0; s < SPT; s++) {
      z[s] = gt.w[s] * gt.S[s];
      segdec[s] *= gt.dec[s];
      if (lane == 0) sDec[wv * SPT + s] = gt.dec[s];
    }
    store_bf16_row<SPT>(sZ + lane * Lds::LDX + wv * SPT, z);
    if (ch + 1 < c_end) {
      const int t1 = t0 + C, rv1 = min(C, T_len - t1);
      pk.load(kb + (size_t)t1 * DK, rv1, tid);
      pv.load(vb + (size_t)t1 * DV, rv1, tid);
      pg.load(gb + (size_t)(t1 + min(lane, rv1 - 1)) * M, lane < rv1);
    }
    __syncthreads();
    W.carry(sK, Lds::LDQ, sV, Lds::LDV, sZ, Lds::LDX, sDec, wv, lane);
    __syncthreads();
  }
  W.store_w(ws_state + ((size_t)unit * P + seg) * M * (DK + DV), wv, lane);
  if (lane == 0) {
#pragma unroll
    for (int s = 0; s < SPT; s++) ws_dec[((size_t)unit * P + seg) * M + wv * SPT + s] = segdec[s];
  }
}

// ----------------------------------------------------- phase B: scan
// One thread per (unit, state element), serial over the segments; the loads of
// a batch of maps are issued before any of the batch's stores.  Slot p holds
// segment p's map on entry (p < P-1) and its start state on exit.
template <int DK, int DV, int M>
__global__ void __launch_bounds__(256)
gsa_bf16_scan(float* __restrict__ ws_state, const float* __restrict__ ws_dec,
              const float* __restrict__ k0, const float* __restrict__ v0, int units, int P) {
  constexpr int NE = M * (DK + DV);
  constexpr int BATCH = 8;
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long long)units * NE) return;
  const int unit = (int)(gid / NE), e = (int)(gid % NE);
  const int c = e / (DK + DV), cl = e % (DK + DV);
  float W = 0.f;
  if (cl < DK) {
    if (k0) W = k0[((size_t)unit * M + c) * DK + cl];
  } else {
    if (v0) W = v0[((size_t)unit * M + c) * DV + cl - DK];
  }
  float* st = ws_state + (size_t)unit * P * NE + e;
  const float* dc = ws_dec + (size_t)unit * P * M + c;
  for (int p0 = 0; p0 + 1 < P; p0 += BATCH) {
    float x[BATCH], d[BATCH];
#pragma unroll
    for (int i = 0; i < BATCH; i++) {
      if (p0 + i + 1 < P) {
        x[i] = st[(size_t)(p0 + i) * NE];
        d[i] = dc[(size_t)(p0 + i) * M];
      }
    }
#pragma unroll
    for (int i = 0; i < BATCH; i++) {
      if (p0 + i + 1 < P) {
        st[(size_t)(p0 + i) * NE] = W;
        W = d[i] * W + x[i];
      }
    }
  }
  st[(size_t)(P - 1) * NE] = W;
}

// ------------------------------------------------------ phase C: outputs
template <int DK, int DV, int M>
__global__ void __launch_bounds__(NT, 1)
gsa_bf16_out(const bf16_t* __restrict__ qq, const bf16_t* __restrict__ kk,
             const bf16_t* __restrict__ vv, const bf16_t* __restrict__ gg,
             const float* __restrict__ k0, const float* __restrict__ v0,
             const float* __restrict__ ws_state, bf16_t* __restrict__ oo, float* __restrict__ kf,
             float* __restrict__ vf, int T_len, int S, int P, float inv_tau) {
  using Lds = OutLds<DK, DV, M>;
  using ST = StateTiles<DK, DV, M, 4>;
  constexpr int SPT = M / NW;
  constexpr int MT = M / 16;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  bf16_t* sQ = reinterpret_cast<bf16_t*>(smem + Lds::oQ);
  bf16_t* sK = reinterpret_cast<bf16_t*>(smem + Lds::oK);
  bf16_t* sV = reinterpret_cast<bf16_t*>(smem + Lds::oV);
  bf16_t* sW = reinterpret_cast<bf16_t*>(smem + Lds::oW);
  bf16_t* sX = reinterpret_cast<bf16_t*>(smem + Lds::oX);
  bf16_t* sZ = reinterpret_cast<bf16_t*>(smem + Lds::oZ);
  float* sE = reinterpret_cast<float*>(smem + Lds::oE);
  float* sDec = reinterpret_cast<float*>(smem + Lds::oDec);

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const bool is_state = wv >= 4;
  const int sw = wv - 4;
  const int seg = blockIdx.x, unit = blockIdx.y;
  const int nchunks = (T_len + C - 1) / C;
  const int c_begin = seg * S, c_end = min(c_begin + S, nchunks);
  const size_t ub = (size_t)unit * T_len;
  const bf16_t* qb = qq + ub * DK;
  const bf16_t* kb = kk + ub * DK;
  const bf16_t* vb = vv + ub * DV;
  const bf16_t* gb = gg + ub * M + wv * SPT;
  bf16_t* ob = oo + ub * DV;

  ST W;
  if (is_state) {
    if (P > 1) W.load_w(ws_state + ((size_t)unit * P + seg) * M * (DK + DV), sw, lane);
    else W.load_kv(k0 ? k0 + (size_t)unit * M * DK : nullptr, v0 ? v0 + (size_t)unit * M * DV : nullptr, sw, lane);
    W.store_copy(sW, Lds::LDW, sw, lane);
  }

  Tile<DK> pq, pk;
  Tile<DV> pv;
  GateRow<SPT> pg;
  {
    const int t0 = c_begin * C, rv = min(C, T_len - t0);
    pq.load(qb + (size_t)t0 * DK, rv, tid);
    pk.load(kb + (size_t)t0 * DK, rv, tid);
    pv.load(vb + (size_t)t0 * DV, rv, tid);
    pg.load(gb + (size_t)(t0 + min(lane, rv - 1)) * M, lane < rv);
  }

  for (int ch = c_begin; ch < c_end; ch++) {
    const int t0 = ch * C, rv = min(C, T_len - t0);
    pq.store(sQ, Lds::LDQ, tid);
    pk.store(sK, Lds::LDQ, tid);
    pv.store(sV, Lds::LDV, tid);
    bool small = false;
    {
      LogGates<SPT> gt;
      gt.compute(pg, lane < rv, inv_tau, lane);
      float x[SPT], z[SPT], e[SPT];
#pragma unroll
      for (int s = 0; s < SPT; s++) {
        const float gc = __shfl(gt.G[s], 63, 64);
        small |= !(gc >= kFastMinLogDecay);
        e[s] = __expf(gt.G[s]);
        x[s] = gt.w[s] * __expf(-gt.G[s]);
        z[s] = gt.w[s] * __expf(gc - gt.G[s]);
        if (lane == 0) sDec[wv * SPT + s] = __expf(gc);
      }
      // the fast-path factors; a slow chunk overwrites this region after the barrier
      store_bf16_row<SPT>(sX + lane * Lds::LDX + wv * SPT, x);
      store_bf16_row<SPT>(sZ + lane * Lds::LDX + wv * SPT, z);
      store_f32_row<SPT>(sE + lane * Lds::LDE + wv * SPT, e);
    }
    GateRow<SPT> pg_next;  // the current row stays in pg for a slow chunk
    if (ch + 1 < c_end) {  // prefetch the next chunk into registers
      const int t1 = t0 + C, rv1 = min(C, T_len - t1);
      pq.load(qb + (size_t)t1 * DK, rv1, tid);
      pk.load(kb + (size_t)t1 * DK, rv1, tid);
      pv.load(vb + (size_t)t1 * DV, rv1, tid);
      pg_next.load(gb + (size_t)(t1 + min(lane, rv1 - 1)) * M, lane < rv1);
    }
    const bool slow = __syncthreads_or(small) != 0;

    if (!slow) {
      if (!is_state) {
        // pass waves hold no state: dropping it frees these registers for the passes
        W.zero();
        pass_chunk<DK, DV, M>(wv, lane, sQ, sK, sV, sW, sX, sE, ob + (size_t)t0 * DV, rv);
      } else {
        W.carry(sK, Lds::LDQ, sV, Lds::LDV, sZ, Lds::LDX, sDec, sw, lane);
      }
    } else {
      // ---- exact token recurrence (no division by a decay product), on an
      // fp32 copy of the state in LDS; thread t owns slot t / TPS and 1/TPS of
      // its columns for the whole chunk
      exact_chunk<DK, DV, M>(W, pg, rv, inv_tau, smem, sQ, sK, sV, ob + (size_t)t0 * DV, tid);
    }
    __syncthreads();
    if (is_state) W.store_copy(sW, Lds::LDW, sw, lane);
    pg = pg_next;
  }

  if (seg == P - 1 && is_state)
    W.store_kv(kf ? kf + (size_t)unit * M * DK : nullptr, vf ? vf + (size_t)unit * M * DV : nullptr, sw, lane);
}

// ------------------------------------------------------------ launcher
template <int DK, int DV, int M>
static int launch(const GsaLaunch& a) {
  using LO = OutLds<DK, DV, M>;
  using LS = StateLds<DK, DV, M>;
  const int units = a.B * a.H;
  const int nchunks = (a.T + C - 1) / C;
  const int S = a.chunks_per_seg;
  const int P = (nchunks + S - 1) / S;
  const float inv_tau = 1.0f / a.tau;
  hipStream_t st = (hipStream_t)a.stream;
  static const bool lds_set = [] {  // once per instantiation and process
    hipFuncSetAttribute((const void*)gsa_bf16_out<DK, DV, M>,
                        hipFuncAttributeMaxDynamicSharedMemorySize, LO::total);
    hipFuncSetAttribute((const void*)gsa_bf16_state<DK, DV, M>,
                        hipFuncAttributeMaxDynamicSharedMemorySize, LS::total);
    return true;
  }();
  (void)lds_set;
  record_event(a.events, 0, a.stream);
  if (P > 1) {
    hipLaunchKernelGGL((gsa_bf16_state<DK, DV, M>), dim3(P - 1, units), dim3(NT), LS::total, st,
                       (const bf16_t*)a.k, (const bf16_t*)a.v, (const bf16_t*)a.g, a.ws_state,
                       a.ws_dec, a.T, S, P, inv_tau);
    record_event(a.events, 1, a.stream);
    const long long ne = (long long)units * M * (DK + DV);
    hipLaunchKernelGGL((gsa_bf16_scan<DK, DV, M>), dim3((unsigned)((ne + 255) / 256)), dim3(256), 0, st,
                       a.ws_state, (const float*)a.ws_dec, a.k0, a.v0, units, P);
  } else {
    record_event(a.events, 1, a.stream);
  }
  record_event(a.events, 2, a.stream);
  hipLaunchKernelGGL((gsa_bf16_out<DK, DV, M>), dim3(P, units), dim3(NT), LO::total, st,
                     (const bf16_t*)a.q, (const bf16_t*)a.k, (const bf16_t*)a.v, (const bf16_t*)a.g,
                     a.k0, a.v0, (const float*)a.ws_state, (bf16_t*)a.o, a.kf, a.vf, a.T, S, P, inv_tau);
  record_event(a.events, 3, a.stream);
  return 0;
}

}  // namespace bfk

#define GSA_BF16_CASE(DKC, DVC, MC)                                      \
  if (dk == DKC && dv == DVC && m == MC) {                                \
    static_assert(bfk::OutLds<DKC, DVC, MC>::total <= kLdsBytes, "LDS"); \
    if (query) return bfk::OutLds<DKC, DVC, MC>::total;                   \
    return bfk::launch<DKC, DVC, MC>(*a);                                 \
  }

// Returns: query -> LDS bytes (>0) or -1 if unsupported; launch -> 0 or -1.
int gsa_dispatch_bf16(int dk, int dv, int m, const GsaLaunch* a, bool query) {
  GSA_BF16_CASE(128, 128, 64)
  GSA_BF16_CASE(128, 128, 32)
  GSA_BF16_CASE(64, 64, 64)
  GSA_BF16_CASE(64, 64, 32)
  return -1;
}

}  // namespace gsa
