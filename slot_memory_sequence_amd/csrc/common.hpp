// Device helpers shared by the libgsa kernels (gfx950 / CDNA4, wave64).
//
// MFMA fragment conventions (checked on gfx950 with an in-bounds lane probe):
//   v_mfma_f32_16x16x32_bf16: lane l holds A[l%16][8*(l/16)+j] and
//   B[8*(l/16)+j][l%16] (j = 0..7) and receives D[4*(l/16)+i][l%16] (i = 0..3).
//   v_mfma_f32_16x16x4_f32: lane l holds A[l%16][l/16], B[l/16][l%16]; same D.
//   ds_read_tr16_b64: inside each 16-lane group, lane i receives element i%4 of
//   the 4-element vector addressed by lane 4*jj + i/4 (jj = 0..3).  Pointing
//   lane L at row (k0 + L/4), column (n0 + 4*(L%4)) of a row-major [k][n] tile
//   therefore delivers tile[k0 + jj][n0 + i] to lane i: a 4(k) x 16(n) block
//   transposed into MFMA operand order, with no transposed copy in LDS.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gsa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_raw;
typedef uint16_t bf16_t;  // bf16 storage as raw bits

#define GSA_LDS __attribute__((address_space(3)))

__device__ __forceinline__ float bf2f(bf16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ __forceinline__ bf16_t f2bf(float x) {
  // round to nearest even; NaN stays NaN
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)((u >> 16) | 0x40);
  return (bf16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// ---------------------------------------------------------------- element IO
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float ld(const float* p) { return *p; }
  static __device__ __forceinline__ float to_f(float x) { return x; }
  static __device__ __forceinline__ float from_f(float x) { return x; }
};
template <> struct Elem<bf16_t> {
  static __device__ __forceinline__ float to_f(bf16_t x) { return bf2f(x); }
  static __device__ __forceinline__ bf16_t from_f(float x) { return f2bf(x); }
};

// ------------------------------------------------------------ MFMA wrappers
// Op<T>: one 16x16 output tile, K-step KS, fragment type Frag.
template <typename T> struct Op;

template <> struct Op<bf16_t> {
  static constexpr int KS = 32;
  typedef bf16x8 Frag;
  static __device__ __forceinline__ f32x4 mma(const Frag& a, const Frag& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  // operand stored [row][k] (k contiguous), leading dim ld (elements)
  static __device__ __forceinline__ Frag ld_k(const bf16_t* base, int ld, int row0, int k0, int lane) {
    const bf16_t* p = base + (row0 + (lane & 15)) * ld + k0 + 8 * (lane >> 4);
    return *reinterpret_cast<const bf16x8*>(p);
  }
  // operand stored [k][row] (row contiguous): transposing LDS read
  static __device__ __forceinline__ Frag ld_t(const bf16_t* base, int ld, int row0, int k0, int lane) {
    const int L = lane & 15, G = lane >> 4;
    const bf16_t* p0 = base + (k0 + 8 * G + (L >> 2)) * ld + row0 + 4 * (L & 3);
    const bf16_t* p1 = p0 + 4 * ld;
    bf16x4_raw lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((GSA_LDS bf16x4_raw*)(p0));
    bf16x4_raw hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((GSA_LDS bf16x4_raw*)(p1));
    Frag f;
    f[0] = lo[0]; f[1] = lo[1]; f[2] = lo[2]; f[3] = lo[3];
    f[4] = hi[0]; f[5] = hi[1]; f[6] = hi[2]; f[7] = hi[3];
    return f;
  }
};

template <> struct Op<float> {
  static constexpr int KS = 4;
  typedef float Frag;
  static __device__ __forceinline__ f32x4 mma(const Frag& a, const Frag& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ Frag ld_k(const float* base, int ld, int row0, int k0, int lane) {
    return base[(row0 + (lane & 15)) * ld + k0 + (lane >> 4)];
  }
  static __device__ __forceinline__ Frag ld_t(const float* base, int ld, int row0, int k0, int lane) {
    return base[(k0 + (lane >> 4)) * ld + row0 + (lane & 15)];
  }
};

// Row padding (elements) for LDS tiles: 16 bytes per row.
template <typename T> struct Pad { static constexpr int v = 16 / sizeof(T); };

// ------------------------------------------------------------- gate math
// log alpha = log sigmoid(g) / tau (stable split), alpha = exp(log alpha),
// write intensity 1 - alpha = -expm1(log alpha).  g = +inf -> (1, 0);
// g = -inf -> (0, 1).
__device__ __forceinline__ void gate_alpha_w(float g, float inv_tau, float& a, float& w) {
  float ls = fminf(g, 0.f) - log1pf(__expf(-fabsf(g)));
  float la = ls * inv_tau;
  a = __expf(la);
  w = -expm1f(la);
}

__device__ __forceinline__ float gate_alpha(float g, float inv_tau) {
  float ls = fminf(g, 0.f) - log1pf(__expf(-fabsf(g)));
  return __expf(ls * inv_tau);
}

// reductions inside 16-lane rows of a wave (lanes sharing l/16)
__device__ __forceinline__ float max16(float x) {
  x = fmaxf(x, __shfl_xor(x, 8, 64));
  x = fmaxf(x, __shfl_xor(x, 4, 64));
  x = fmaxf(x, __shfl_xor(x, 2, 64));
  x = fmaxf(x, __shfl_xor(x, 1, 64));
  return x;
}
__device__ __forceinline__ float sum16(float x) {
  x += __shfl_xor(x, 8, 64);
  x += __shfl_xor(x, 4, 64);
  x += __shfl_xor(x, 2, 64);
  x += __shfl_xor(x, 1, 64);
  return x;
}
__device__ __forceinline__ float sum64(float x) {
  x += __shfl_xor(x, 32, 64);
  x += __shfl_xor(x, 16, 64);
  return sum16(x);
}
__device__ __forceinline__ float sum32(float x) {
  x += __shfl_xor(x, 16, 64);
  return sum16(x);
}

// Threshold for the single-reference chunk factorisation: every slot's
// whole-chunk decay product must stay >= e^-40 so that 1/prod stays <= e^40.
constexpr float kFastMinDecay = 4.248354255291589e-18f;  // e^-40

// ------------------------------------------------------------ gate input
// How the GLA forward's gate tensor is given: as logits, alpha =
// sigmoid(g)^(1/tau) (Sec. 2.3 / 3.3), or directly as per-token log-decays,
// log alpha = min(g, 0) (a gate vector computed elsewhere).  The values match
// the GSA_GATE_* codes of the C ABI.
enum GateMode : int { kGateLogit = 0, kGateLogDecay = 1 };

// ------------------------------------------------- slot read non-linearity
// What turns the pass-1 slot scores o'_t into the pass-2 read weights s_t: the
// softmax over the m slots (Sec. 3.2), or one of the element-wise functions
// the ablation study puts in its place (Table 2: no non-linearity, Swish, ReLU,
// ReLU^2).  The values match the GSA_SLOT_* codes of the C ABI.
enum SlotAct : int { kActSoftmax = 0, kActIdentity = 1, kActSwish = 2, kActRelu = 3, kActRelu2 = 4 };

// The element-wise replacements (not used for kActSoftmax, which needs the
// whole slot row).  Swish(x) = x * sigmoid(x), formed as x / (1 + e^-x): for
// x -> -inf the quotient goes to -0, never inf * 0.
template <int ACT>
__device__ __forceinline__ float slot_act(float x) {
  static_assert(ACT >= kActIdentity && ACT <= kActRelu2, "element-wise slot non-linearity");
  if constexpr (ACT == kActIdentity) return x;
  else if constexpr (ACT == kActSwish) return x / (1.f + __expf(-x));
  else if constexpr (ACT == kActRelu) return fmaxf(x, 0.f);
  else {
    const float r = fmaxf(x, 0.f);
    return r * r;
  }
}

// Their derivatives (the backward's dz = f'(z) ds): 1; sigmoid(x) (1 + x (1 -
// sigmoid(x))); the step x > 0; 2 max(x, 0).
template <int ACT>
__device__ __forceinline__ float slot_act_grad(float x) {
  static_assert(ACT >= kActIdentity && ACT <= kActRelu2, "element-wise slot non-linearity");
  if constexpr (ACT == kActIdentity) return 1.f;
  else if constexpr (ACT == kActSwish) {
    const float sg = 1.f / (1.f + __expf(-x));
    return sg * (1.f + x * (1.f - sg));
  } else if constexpr (ACT == kActRelu) return x > 0.f ? 1.f : 0.f;
  else return x > 0.f ? 2.f * x : 0.f;
}

}  // namespace gsa
