// bf16 building blocks shared by the chunkwise GSA and GLA kernels (gfx950):
// MFMA wrappers and operand fragment loads from LDS, chunk tile I/O, raw
// bf16 rows, wave-wide DPP scans and the log2-domain gate.
#pragma once
#include "common.hpp"
#include "internal.hpp"

namespace gsa {
namespace bfk {

constexpr int C = 64;   // chunk length
constexpr int NW = 8;   // waves per workgroup
constexpr int NT = NW * 64;
// log2 of the smallest decay the factorised forms allow between a token and
// its reference point: over a whole chunk in the chunk form, over a 16-token
// sub-chunk in the forward's sub-chunk form (2^-90, about e^-62).  The forms
// divide by the decay E from the reference point, so X = (1 - alpha) / E <=
// 2^90: a masked score times X stays about 2^38 below
// the bf16 / fp32 overflow at 2^128 (no inf to meet a zero mask), E stays a
// normal fp32 number, and every product that survives the causal mask is a
// ratio E_j / E_r <= 1 formed from two factors of exact relative precision.
constexpr float kFastMinLog2Decay = -90.0f;
// Up to this many segment maps before the last segment, the output workgroups
// build their start states from the maps themselves (no scan launch).
constexpr int kMaxFoldedMaps = 3;

typedef __attribute__((ext_vector_type(8))) float f32x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4v;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;

__device__ __forceinline__ f32x4 mma(const bf16x8& a, const bf16x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16x16x16 product (one 16-row sub-chunk as the contraction) as a 16x16x32
// one whose second half of the contraction is zero on both operands (lane
// group g's four values take contraction positions 8g .. 8g + 3).  The
// 16x16x16 bf16 instruction itself (v_mfma_f32_16x16x16_bf16) was measured
// to give wrong accumulators in one schedule of the backward kernel (its
// first pass wave at dk = dv = 128, m = 64, where the product's result is
// read soon after a 16x16x32 one), while this form gave the expected ones.
__device__ __forceinline__ f32x4 mma16(const bf16x4v& a, const bf16x4v& b, f32x4 c) {
  const __bf16 z = (__bf16)0.f;
  const bf16x8 a8 = {a[0], a[1], a[2], a[3], z, z, z, z};
  const bf16x8 b8 = {b[0], b[1], b[2], b[3], z, z, z, z};
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, b8, c, 0, 0, 0);
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

// Row-major [k][n] tile read column-wise, four k (k0 already includes the lane
// group's offset): lane l gets tile[k0 + jj][n0 + l%16], jj = 0..3 (the
// 16x16x16 operand order).
__device__ __forceinline__ bf16x4v ld_col4(const bf16_t* base, int ld, int n0, int k0, int lane) {
  const int L = lane & 15;
  const bf16_t* p0 = base + (k0 + (L >> 2)) * ld + n0 + 4 * (L & 3);
  bf16x4_raw lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((GSA_LDS bf16x4_raw*)(p0));
  return bf16x4v{lo[0], lo[1], lo[2], lo[3]};
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

// ------------------------------------------------------- global tile I/O
// [C][D] bf16 chunk tile moved as 16-byte vectors by the 512 threads.
template <int D>
struct Tile {
  static constexpr int VPR = D / 8;
  static constexpr int NV = C * VPR / NT;
  static_assert(NV >= 1 && (C * VPR) % NT == 0, "tile/thread mismatch");
  uint4 r[NV];
  // rows >= rows_valid (>= 1) read the last valid row; store() zeroes them, so
  // the loads are not waited for until the tile is stored
  __device__ __forceinline__ void load(const bf16_t* __restrict__ base, int rows_valid, int tid) {
#pragma unroll
    for (int i = 0; i < NV; i++) {
      const int idx = tid + NT * i, row = idx / VPR, cv = idx % VPR;
      r[i] = *reinterpret_cast<const uint4*>(base + min(row, rows_valid - 1) * D + cv * 8);
    }
  }
  __device__ __forceinline__ void store(bf16_t* dst, int ld, int rows_valid, int tid) const {
#pragma unroll
    for (int i = 0; i < NV; i++) {
      const int idx = tid + NT * i, row = idx / VPR, cv = idx % VPR;
      const bool ok = row < rows_valid;
      *reinterpret_cast<uint4*>(dst + row * ld + cv * 8) =
          make_uint4(ok ? r[i].x : 0u, ok ? r[i].y : 0u, ok ? r[i].z : 0u, ok ? r[i].w : 0u);
    }
  }
  // The same with a uniform branch for full tiles (no row clamp, no zeroing):
  // fewer vector instructions, for kernels whose waits do not depend on the
  // loads being branch-free (the output kernels' prefetches do).
  __device__ __forceinline__ void load_branchy(const bf16_t* __restrict__ base, int rows_valid, int tid) {
    if (rows_valid >= C) {
#pragma unroll
      for (int i = 0; i < NV; i++) r[i] = *reinterpret_cast<const uint4*>(base + (size_t)(tid + NT * i) * 8);
    } else {
      load(base, rows_valid, tid);
    }
  }
  __device__ __forceinline__ void store_branchy(bf16_t* dst, int ld, int rows_valid, int tid) const {
    if (rows_valid >= C) {
#pragma unroll
      for (int i = 0; i < NV; i++) {
        const int idx = tid + NT * i, row = idx / VPR, cv = idx % VPR;
        *reinterpret_cast<uint4*>(dst + row * ld + cv * 8) = r[i];
      }
    } else {
      store(dst, ld, rows_valid, tid);
    }
  }
};

// SPT gate logits of one token row (SPT = 4 or 8 bf16 = 8 or 16 bytes).
template <int SPT>
struct GateRow {
  static_assert(SPT >= 2 && SPT % 2 == 0, "gate row width");
  uint32_t r[SPT / 2];
  // p must point at a readable row, 4-byte aligned (the caller clamps the
  // row); rows past the end are masked by the consumer
  __device__ __forceinline__ void load(const bf16_t* __restrict__ p) {
    if constexpr (SPT % 8 == 0) {
#pragma unroll
      for (int i = 0; i < SPT / 8; i++) {
        const uint4 x = reinterpret_cast<const uint4*>(p)[i];
        r[4 * i] = x.x; r[4 * i + 1] = x.y; r[4 * i + 2] = x.z; r[4 * i + 3] = x.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < SPT / 2; i++) r[i] = reinterpret_cast<const uint32_t*>(p)[i];
    }
  }
  __device__ __forceinline__ float at(int s) const {
    const uint32_t w = r[s >> 1];
    return __uint_as_float((s & 1) ? (w & 0xffff0000u) : (w << 16));
  }
  // an opaque redefinition: uses of the row (and the wait for its load) stay
  // after this point
  template <int N = SPT>
  __device__ __forceinline__ void pin() {
#pragma unroll
    for (int i = 0; i < N / 2; i++) asm volatile("" : "+v"(r[i]));
  }
};

// ------------------------------------------------------------- gate math
// All gate quantities are kept in base-2 logarithms so that the hardware
// exp2 / log2 instructions apply directly.

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_zero(float x) {  // DPP lane move, 0 where no source lane
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xf, true));
}

// Inclusive prefix sums over the 64 lanes of a wave, for N independent
// values per lane, step-major so that every step issues N independent
// operations: shifts by 1, 2, 4, 8 inside each row of 16 lanes, then the last
// lane of rows 0 / 2 into rows 1 / 3 and the last lane of row 1 into rows 2, 3.
// wave_row_prefix_sums leaves the inclusive prefix sums inside each row of 16
// lanes; wave_row_carry then adds the totals of the rows before.
template <int N>
__device__ __forceinline__ void wave_row_prefix_sums(float (&x)[N]) {
#pragma unroll
  for (int i = 0; i < N; i++) x[i] += dpp_zero<0x111, 0xf>(x[i]);  // row_shr:1
#pragma unroll
  for (int i = 0; i < N; i++) x[i] += dpp_zero<0x112, 0xf>(x[i]);  // row_shr:2
#pragma unroll
  for (int i = 0; i < N; i++) x[i] += dpp_zero<0x114, 0xf>(x[i]);  // row_shr:4
#pragma unroll
  for (int i = 0; i < N; i++) x[i] += dpp_zero<0x118, 0xf>(x[i]);  // row_shr:8
}
template <int N>
__device__ __forceinline__ void wave_row_carry(float (&x)[N]) {
#pragma unroll
  for (int i = 0; i < N; i++) x[i] += dpp_zero<0x142, 0xa>(x[i]);  // row_bcast:15 into rows 1, 3
#pragma unroll
  for (int i = 0; i < N; i++) x[i] += dpp_zero<0x143, 0xc>(x[i]);  // row_bcast:31 into rows 2, 3
}
template <int N>
__device__ __forceinline__ void wave_prefix_sums(float (&x)[N]) {
  wave_row_prefix_sums<N>(x);
  wave_row_carry<N>(x);
}

// Value of the previous lane of the wave (a whole-wave shift by one lane);
// lane 0 gets `first`.
__device__ __forceinline__ float prev_lane(float x, float first) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(__float_as_int(first), __float_as_int(x), 0x138, 0xf, 0xf, false));
}

// Max / sum of x over lanes l, l^16, l^32, l^48 (the four lane groups of a
// 64-lane wave; every lane gets the result).  gfx950's half-wave and row
// swaps (v_permlane32_swap, v_permlane16_swap), each with one register as both
// operands, give every lane its partner's value in one of the two results,
// so the exchange needs no LDS round trip.
__device__ __forceinline__ float group4_max(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
  const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}
__device__ __forceinline__ float group4_sum(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// log2 alpha = log2(sigmoid(g)) / tau = -log2(1 + 2^-t) / tau with t = g / ln 2,
// clamped at -115 (alpha ~ 2.4e-35) so that g = -inf gives a finite value.
// For t << 0, 2^-t overflows to inf and the clamp applies; for t >> 0 the sum
// rounds to 1 and the result is 0, which is what the split form
// min(t, 0) - log2(1 + 2^-|t|) also gives in fp32 (1 + 2^-|t| rounds the
// same way), at three VALU operations more per gate.
__device__ __forceinline__ float gate_log2(float g, float inv_tau) {
  const float t = g * 1.4426950408889634f;  // g / ln 2
  const float ls2 = -__builtin_amdgcn_logf(1.f + __builtin_amdgcn_exp2f(-t));
  return fmaxf(ls2 * inv_tau, -115.f);
}

// gate_log2 of the token's logit, or exactly 0 (an identity step) for a row past
// the end of the sequence.  The row is masked on the input (g = 1e30 gives
// exp2(-|t|) = 0, log2(1) = 0), so the transcendentals run for every lane and
// the compiler has no reason to branch around them.
__device__ __forceinline__ float gate_log2_or_identity(float g, bool valid, float inv_tau) {
  return gate_log2(valid ? g : 1e30f, inv_tau);
}

// The same for either gate input (GateMode): a logit as above, or a natural
// log-decay taken as given (clamped to [-115 ln 2, 0], so alpha <= 1 and
// -inf is finite); 0 for a row past the end.
template <int GM>
__device__ __forceinline__ float gate_log2_mode(float g, bool valid, float inv_tau) {
  if constexpr (GM == kGateLogit) {
    return gate_log2_or_identity(g, valid, inv_tau);
  } else {
    const float l2 = fmaxf(fminf(g, 0.f) * 1.4426950408889634f, -115.f);
    return valid ? l2 : 0.f;
  }
}

// SPT consecutive bf16 of an LDS row -> floats (p 16-byte aligned when SPT is
// a multiple of 8, else 4-byte aligned)
template <int SPT>
__device__ __forceinline__ void lds_row(const bf16_t* p, float* out) {
  if constexpr (SPT % 8 == 0) {
#pragma unroll
    for (int i = 0; i < SPT; i += 8) {
      const uint4 x = *reinterpret_cast<const uint4*>(p + i);
      const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int j = 0; j < 4; j++) {
        out[i + 2 * j] = __uint_as_float(w[j] << 16);
        out[i + 2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < SPT; i += 2) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(p + i);
      out[i] = __uint_as_float(w << 16);
      out[i + 1] = __uint_as_float(w & 0xffff0000u);
    }
  }
}

// Workgroup-wide OR of a wave-uniform flag: one LDS word per wave and one
// barrier (cheaper than the library's reduction, which takes three barriers).
// flags points at 2 x NW ints; round r uses half r & 1, so a round's writes
// never meet the previous round's reads (every wave reads a round's flags
// before it reaches the next round's barrier).
__device__ __forceinline__ bool block_any(bool wave_flag, int* flags, int round, int lane, int wv) {
  int* f = flags + (round & 1) * NW;
  if (lane == 0) f[wv] = wave_flag ? 1 : 0;
  __syncthreads();
  const int4 a = *reinterpret_cast<const int4*>(f);
  const int4 b = *reinterpret_cast<const int4*>(f + 4);
  return (a.x | a.y | a.z | a.w | b.x | b.y | b.z | b.w) != 0;
}

// Workgroup-wide OR of wave-uniform flag bits, as block_any.
__device__ __forceinline__ int block_or(int wave_flags, int* flags, int round, int lane, int wv) {
  int* f = flags + (round & 1) * NW;
  if (lane == 0) f[wv] = wave_flags;
  __syncthreads();
  const int4 a = *reinterpret_cast<const int4*>(f);
  const int4 b = *reinterpret_cast<const int4*>(f + 4);
  return a.x | a.y | a.z | a.w | b.x | b.y | b.z | b.w;
}

// SPT consecutive floats -> bf16 / fp32 rows in LDS; dst is 4-byte (bf16) /
// 8-byte (fp32) aligned at least, 16-byte when SPT is a multiple of 8 / 4.
template <int SPT>
__device__ __forceinline__ void store_bf16_row(bf16_t* dst, const float* v) {
  if constexpr (SPT % 8 == 0) {
#pragma unroll
    for (int i = 0; i < SPT; i += 8) {
      f32x8 x = {v[i], v[i + 1], v[i + 2], v[i + 3], v[i + 4], v[i + 5], v[i + 6], v[i + 7]};
      *reinterpret_cast<bf16x8*>(dst + i) = __builtin_convertvector(x, bf16x8);
    }
  } else {
    typedef __attribute__((ext_vector_type(2))) float f32x2;
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
#pragma unroll
    for (int i = 0; i < SPT; i += 2) {
      f32x2 x = {v[i], v[i + 1]};
      *reinterpret_cast<bf16x2*>(dst + i) = __builtin_convertvector(x, bf16x2);
    }
  }
}
template <int SPT>
__device__ __forceinline__ void store_f32_row(float* dst, const float* v) {
  if constexpr (SPT % 4 == 0) {
#pragma unroll
    for (int s = 0; s < SPT; s += 4)
      *reinterpret_cast<float4*>(dst + s) = make_float4(v[s], v[s + 1], v[s + 2], v[s + 3]);
  } else {
#pragma unroll
    for (int s = 0; s < SPT; s += 2) *reinterpret_cast<float2*>(dst + s) = make_float2(v[s], v[s + 1]);
  }
}

// Output workgroup -> (segment, unit).  Consecutive workgroup ids are
// dispatched to the eight XCDs in turn (id mod 8).  When the output workgroups
// fold segment maps (fold != 0) and the unit count is a multiple of 8, every
// segment of a unit is placed on one XCD (the ids congruent to the unit mod 8),
// so that the segments of a unit can share its maps in that XCD's L2;
// otherwise the segments of a unit have consecutive ids.
struct SegUnit {
  int seg, unit;
};
__device__ __forceinline__ SegUnit seg_unit(int id, int P, int units, int fold) {
  if (fold && (units & 7) == 0) {
    const int k = id >> 3;
    return {k % P, (id & 7) + 8 * (k / P)};
  }
  return {id % P, id / P};
}

// ------------------------------------------------------------ sequences
// Where the tokens of unit u sit: rows [base, base + len) of the q, k, v, g and
// o arrays, one row per token (row pitch d, so a chunk is one contiguous tile).
struct Span {
  size_t base;
  int len;
};

// A dense batch [B, H, T, d]: unit u = b*H + h holds rows u*T .. u*T + T - 1.
// unit_of maps the launch order of the units to the units (here the identity).
struct DenseSeqs {
  static constexpr bool kVar = false;
  static constexpr int kGroups = 1;  // slot groups per (b, h): see SlotGroups
  int T;
  __device__ __forceinline__ Span span(int unit) const { return {(size_t)unit * T, T}; }
  __device__ __forceinline__ int unit_of(int i) const { return i; }
};

// A packed batch of n variable-length sequences, head-major [H, total, d]:
// sequence s of head h holds rows h*total + cu[s] .. h*total + cu[s+1] - 1 and
// is unit u = s*H + h (the states stay [n, H, m, d]).  Passed by value, so the
// offsets live in the kernel arguments and need no device memory.  The units
// are launched longest sequence first (order[] = the sequences by decreasing
// length), so that the short ones fill the tail of the grid.
struct VarSeqs {
  static constexpr bool kVar = true;
  static constexpr int kGroups = 1;
  int H, total;
  int cu[kMaxVarSeqs + 1];
  int order[kMaxVarSeqs];
  __device__ __forceinline__ Span span(int unit) const {
    const int s = unit / H, h = unit - s * H;
    return {(size_t)h * total + cu[s], cu[s + 1] - cu[s]};
  }
  __device__ __forceinline__ int unit_of(int i) const {
    const int r = i / H;
    return order[r] * H + (i - r * H);
  }
};

// A dense batch whose 2M slots run as two groups of M, each group its own unit
// (the slot rows of K~ and V~ never mix in the recurrence, Sec. 3.2; only the
// read's softmax spans both groups, and it is merged afterwards from each
// group's log-sum-exp).  Unit 2u + h is group h of (b, h) unit u: it reads the
// q, k, v rows of unit u and gate columns hM .. hM + M - 1 of its g rows (row
// pitch 2M), and writes its normalised output rows and log-sum-exps
// interleaved with the other group's ([rows][2][dv], [rows][2]).  Its states
// are slot rows hM .. hM + M - 1 of unit u's, which sit where a unit 2u + h of
// M slots would: no offset changes there.
struct SlotGroups {
  static constexpr bool kVar = false;
  static constexpr int kGroups = 2;
  int T;
  __device__ __forceinline__ Span span(int unit) const { return {(size_t)(unit >> 1) * T, T}; }
  __device__ __forceinline__ int unit_of(int i) const { return i; }
};

// First gate logit of a unit's rows (row pitch M * kGroups) and its group.
template <class Seq, int M>
__device__ __forceinline__ size_t gate_base(const Span& sp, int unit) {
  return sp.base * (M * Seq::kGroups) + (size_t)(unit % Seq::kGroups) * M;
}

}  // namespace bfk
}  // namespace gsa
