// Chunk gate factors and the fp32 slot state held in MFMA accumulators,
// shared by the bf16 GSA forward and backward kernels (gfx950).
#pragma once
#include "bf16_common.hpp"

namespace gsa {
namespace bfk {

// State-map factors: the decay from token r to the chunk end
// S_r = prod_{i>r} alpha_i = exp2(G_C - G_r), the write term
// Z_r = (1 - alpha_r) S_r = S_r - S_{r-1}, and the whole-chunk decay.
template <int SPT>
struct SuffixGates {
  float Z[SPT], dec[SPT];
  __device__ __forceinline__ void compute(const GateRow<SPT>& g, bool valid, float inv_tau) {
    float G[SPT];
#pragma unroll
    for (int s = 0; s < SPT; s++) G[s] = gate_log2_or_identity(g.at(s), valid, inv_tau);
    wave_prefix_sums<SPT>(G);
#pragma unroll
    for (int s = 0; s < SPT; s++) {
      const float tot = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(G[s]), 63));
      dec[s] = __builtin_amdgcn_exp2f(tot);
      Z[s] = __builtin_amdgcn_exp2f(tot - G[s]);
    }
#pragma unroll
    for (int s = 0; s < SPT; s++) Z[s] -= prev_lane(Z[s], dec[s]);
  }
};

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
  // one segment map (layout of load_w) into registers, and the segment step
  // W <- Diag(dec) W + map with the scan kernel's operation order
  typedef f32x4 MapRegs[NCW][MT];
  __device__ __forceinline__ void load_map(MapRegs& x, const float* __restrict__ src, int sw,
                                           int lane) const {
#pragma unroll
    for (int n = 0; n < NCW; n++)
#pragma unroll
      for (int ct = 0; ct < MT; ct++) {
        const float4 v = *reinterpret_cast<const float4*>(
            src + (size_t)(16 * ct + (lane & 15)) * (DK + DV) + col(sw, n, lane));
        x[n][ct] = f32x4{v.x, v.y, v.z, v.w};
      }
  }
  __device__ __forceinline__ void fold(const MapRegs& x, const float* __restrict__ dec, int lane) {
#pragma unroll
    for (int ct = 0; ct < MT; ct++) {
      const float d = dec[16 * ct + (lane & 15)];
#pragma unroll
      for (int n = 0; n < NCW; n++)
#pragma unroll
        for (int i = 0; i < 4; i++) st[n][ct][i] = d * st[n][ct][i] + x[n][ct][i];
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
  }  // the same to global memory with streaming stores: a segment map is read
  // only by the next launch, so its lines need not stay in L2 (less for the
  // end of the kernel to write back)
  __device__ __forceinline__ void store_w_nt(float* __restrict__ dst, int sw, int lane) const {
#pragma unroll
    for (int n = 0; n < NCW; n++)
#pragma unroll
      for (int ct = 0; ct < MT; ct++)
        __builtin_nontemporal_store(
            st[n][ct], reinterpret_cast<f32x4*>(dst + (size_t)(16 * ct + (lane & 15)) * (DK + DV) + col(sw, n, lane)));
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
  // W^T <- W^T Diag(dec) + [A | B]^T [Za | Zb] over one chunk: the first DK
  // state columns take A's columns with Za, the others B's columns with Zb
  // (A, B [C][lda|ldb], Za, Zb [C][ldz], bf16); dec nullable (no decay).
  __device__ __forceinline__ void update2(const bf16_t* sA, int lda, const bf16_t* sB, int ldb,
                                          const bf16_t* sZa, const bf16_t* sZb, int ldz,
                                          const float* sDec, int sw, int lane) {
    const int L = lane & 15, g = lane >> 4;
    if (sDec) {
#pragma unroll
      for (int ct = 0; ct < MT; ct++) {
        const float d = sDec[16 * ct + L];
#pragma unroll
        for (int n = 0; n < NCW; n++)
#pragma unroll
          for (int i = 0; i < 4; i++) st[n][ct][i] *= d;
      }
    }
    // a wave's columns lie in one half (static_assert above), so the choice is wave-uniform
    const bool khalf = 16 * (sw * NCW) < DK;
    const bf16_t* sZ = khalf ? sZa : sZb;
#pragma unroll
    for (int r0 = 0; r0 < C; r0 += 32) {
      bf16x8 zb[MT];
#pragma unroll
      for (int ct = 0; ct < MT; ct++) zb[ct] = ld_col(sZ, ldz, 16 * ct, r0 + 8 * g, r0 + 8 * g + 4, lane);
#pragma unroll
      for (int n = 0; n < NCW; n++) {
        const int c0 = 16 * (sw * NCW + n);
        const bf16x8 a = khalf ? ld_col(sA, lda, c0, r0 + 8 * g, r0 + 8 * g + 4, lane)
                               : ld_col(sB, ldb, c0 - DK, r0 + 8 * g, r0 + 8 * g + 4, lane);
#pragma unroll
        for (int ct = 0; ct < MT; ct++) st[n][ct] = mma(a, zb[ct], st[n][ct]);
      }
    }
  }
  // update2 in the sub-chunk form (chunk_factors): Za, Zb hold weights at the
  // reference point of each token's 16-token sub-chunk T, and sD [4][M] the
  // decays between reference points.  A lane's eight contraction values (8
  // consecutive tokens) lie in one sub-chunk T and one slot c, so its Z
  // operand is carried to the chunk start by the one factor sD[0][c] * ... *
  // sD[T-1][c] and the update is update2's.
  __device__ __forceinline__ void update2_sub(const bf16_t* sA, int lda, const bf16_t* sB, int ldb,
                                              const bf16_t* sZa, const bf16_t* sZb, int ldz,
                                              const float* sDec, const float* sD, int sw, int lane) {
    const int L = lane & 15, g = lane >> 4;
#pragma unroll
    for (int ct = 0; ct < MT; ct++) {
      const float d = sDec[16 * ct + L];
#pragma unroll
      for (int n = 0; n < NCW; n++)
#pragma unroll
        for (int i = 0; i < 4; i++) st[n][ct][i] *= d;
    }
    const bool khalf = 16 * (sw * NCW) < DK;
    const bf16_t* sZ = khalf ? sZa : sZb;
#pragma unroll
    for (int r0 = 0; r0 < C; r0 += 32) {
      bf16x8 zb[MT];
#pragma unroll
      for (int ct = 0; ct < MT; ct++) {
        // tokens r0 + 8g .. r0 + 8g + 7: sub-chunk T = r0 / 16 + g / 2
        const int c = 16 * ct + L;
        float f = g >= 2 ? sD[(r0 / 16) * M + c] : 1.f;
        if (r0 == 32) f *= sD[c] * sD[M + c];
        f32x8 z = __builtin_convertvector(ld_col(sZ, ldz, 16 * ct, r0 + 8 * g, r0 + 8 * g + 4, lane), f32x8);
#pragma unroll
        for (int i = 0; i < 8; i++) z[i] *= f;
        zb[ct] = __builtin_convertvector(z, bf16x8);
      }
#pragma unroll
      for (int n = 0; n < NCW; n++) {
        const int c0 = 16 * (sw * NCW + n);
        const bf16x8 a = khalf ? ld_col(sA, lda, c0, r0 + 8 * g, r0 + 8 * g + 4, lane)
                               : ld_col(sB, ldb, c0 - DK, r0 + 8 * g, r0 + 8 * g + 4, lane);
#pragma unroll
        for (int ct = 0; ct < MT; ct++) st[n][ct] = mma(a, zb[ct], st[n][ct]);
      }
    }
  }
};


// ------------------------------------------------------ chunk factors
// Regime bits of a chunk, OR-ed over its slots and then over the workgroup.
constexpr int kNeedSub = 1;    // some slot decays below 2^-90 over the chunk
constexpr int kNeedExact = 2;  // ... over one of its 16-token sub-chunks

// SPT slots from slot0 of one chunk (token row = lane) into one factor set:
// Z = (1-alpha_r) prod_{i>r} alpha_i, E and X = (1-alpha) / E, four decay rows
// d[0..3] and the whole-chunk decay.  A slot whose chunk decay stays in the
// factorised range gets the chunk-local E and X (cumulative from the chunk
// start, the one reference point): d[0..2] = 1 between its coinciding
// reference points and d[3] = the chunk decay after the last of them.  Any
// other slot gets sub-chunk reference points (GSA paper App. A.1, the
// secondary chunking) at tokens 0, 16, 32, 48: E and X cumulative from the
// start of the token's own 16-token sub-chunk, and d[R] = the decay across
// sub-chunk R.  A term between a token of sub-chunk R and a later one of
// sub-chunk J then carries d[R] * ... * d[J-1] (the state at the chunk start
// counts as reference point 0, the chunk end as the point after d[3]); its Z
// comes from suffix products (no division).  Both representations give the
// same results under the sub-chunk form, and a chunk in which no slot needs
// the second one can use the plain chunk form.  E also returns this lane's E.
// Returns the regime bits of these slots.
template <int SPT, int LDX, int LDE, int M, class Row>
__device__ __forceinline__ int chunk_factors(const Row& g, bool valid, float inv_tau,
                                             int lane, int slot0, bf16_t* sX, bf16_t* sZ, float* sE,
                                             float* sD, float* sDec, float (&E)[SPT]) {
  float G[SPT], Gl[SPT];
#pragma unroll
  for (int s = 0; s < SPT; s++) G[s] = gate_log2_or_identity(g.at(s), valid, inv_tau);
  wave_row_prefix_sums<SPT>(G);
#pragma unroll
  for (int s = 0; s < SPT; s++) Gl[s] = G[s];  // sums inside the lane's sub-chunk
  wave_row_carry<SPT>(G);
  float X[SPT], z[SPT], gc[SPT];
  bool any = false;
#pragma unroll
  for (int s = 0; s < SPT; s++) {
    gc[s] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(G[s]), 63));
    any |= !(gc[s] >= kFastMinLog2Decay);
    E[s] = __builtin_amdgcn_exp2f(G[s]);
    X[s] = __builtin_amdgcn_exp2f(-G[s]);
  }
#pragma unroll
  for (int s = 0; s < SPT; s++) X[s] -= prev_lane(X[s], 1.f);
  float d[SPT];  // this lane's entry of the d rows (lanes 0..3)
#pragma unroll
  for (int s = 0; s < SPT; s++) {
    const float dc = __builtin_amdgcn_exp2f(gc[s]);
    z[s] = X[s] * dc;
    d[s] = lane == 3 ? dc : 1.f;
    if (lane == 0) sDec[slot0 + s] = dc;
  }
  int flags = 0;
  if (any) {  // wave-uniform: some slot of this wave leaves the chunk-local range
#pragma unroll
    for (int s = 0; s < SPT; s++) {
      if (gc[s] >= kFastMinLog2Decay) continue;  // uniform
      flags |= kNeedSub;
      const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(Gl[s]), 15));
      const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(Gl[s]), 31));
      const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(Gl[s]), 47));
      const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(Gl[s]), 63));
      if (!(fminf(fminf(r0, r1), fminf(r2, r3)) >= kFastMinLog2Decay)) flags |= kNeedExact;
      E[s] = __builtin_amdgcn_exp2f(Gl[s]);
      const float xi = __builtin_amdgcn_exp2f(-Gl[s]);
      const float xp = prev_lane(xi, 1.f);
      X[s] = xi - ((lane & 15) ? xp : 1.f);
      // S_r = prod_{i>r} alpha_i = 2^(G_C - G_r); Z_r = S_r - S_{r-1}, S_{-1} = chunk decay
      const float sr = __builtin_amdgcn_exp2f(gc[s] - G[s]);
      z[s] = sr - prev_lane(sr, __builtin_amdgcn_exp2f(gc[s]));
      d[s] = __builtin_amdgcn_exp2f(lane == 0 ? r0 : lane == 1 ? r1 : lane == 2 ? r2 : r3);
    }
  }
  store_bf16_row<SPT>(sX + lane * LDX + slot0, X);
  store_bf16_row<SPT>(sZ + lane * LDX + slot0, z);
  store_f32_row<SPT>(sE + lane * LDE + slot0, E);
  if (lane < 4) store_f32_row<SPT>(sD + lane * M + slot0, d);
  return flags;
}

}  // namespace bfk
}  // namespace gsa
