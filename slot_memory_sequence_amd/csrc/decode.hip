// One recurrent GSA step for a batch of sequences (single-token decode).
//
// Method: "Gated Slot Attention for Efficient Linear-Time Sequence Modeling",
// Sec. 3.2 (per-slot gated RNN, recurrent form of Fig. 2) and Sec. 3.3 (forget
// gate sigmoid(g)^(1/tau)).  For every (sequence, head), in place:
//   Kt <- Diag(a) Kt + (1-a) k^T ;  s = softmax(Kt q) ;
//   Vt <- Diag(a) Vt + (1-a) v^T ;  o = Vt^T s.
// The softmax may be replaced by one of the element-wise functions of the
// paper's ablation study (Table 2), selected by the ACT template parameter.
// The step is bound by HBM traffic: the two fp32 slot states are read and
// written once (2 * 2 * m * d * 4 bytes per unit) while the token I/O is tiny,
// the reason the paper ties inference speed to state size (Sec. 4.1.4).
//
// Layout: one workgroup per unit; each thread owns NK float4 of Kt and of Vt
// (row c = f / (DK/4)), all loaded before any arithmetic so that the unit's
// whole state (64 KB at m = 64, d = 128) is in flight at once.
#include "common.hpp"
#include "internal.hpp"
#include "launch.hpp"

namespace gsa {


template <typename T>
__device__ __forceinline__ void load4(const T* p, float* out);
template <>
__device__ __forceinline__ void load4<float>(const float* p, float* out) {
  float4 x = *reinterpret_cast<const float4*>(p);
  out[0] = x.x; out[1] = x.y; out[2] = x.z; out[3] = x.w;
}
template <>
__device__ __forceinline__ void load4<bf16_t>(const bf16_t* p, float* out) {
  uint2 x = *reinterpret_cast<const uint2*>(p);
  out[0] = __uint_as_float(x.x << 16);
  out[1] = __uint_as_float(x.x & 0xffff0000u);
  out[2] = __uint_as_float(x.y << 16);
  out[3] = __uint_as_float(x.y & 0xffff0000u);
}
template <typename T>
__device__ __forceinline__ void store4(T* p, const float* v);
template <>
__device__ __forceinline__ void store4<float>(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t* p, const float* v) {
  uint2 x;
  x.x = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
  x.y = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
  *reinterpret_cast<uint2*>(p) = x;
}

// float4 of each state per thread (8: 256 threads for m = 64, d = 128) and
// non-temporal state loads / stores: the fastest pair measured on MI355X for
// this read-modify-write stream (about 6.1 TB/s, against 5.4 TB/s for plain
// loads and stores and 5.3-6.0 TB/s for 512 or 1024 threads per unit)
#ifndef GSA_DECODE_KPER
#define GSA_DECODE_KPER 8
#endif
#ifndef GSA_DECODE_NT
#define GSA_DECODE_NT 1
#endif

// The states are streamed once: non-temporal loads and stores keep them from
// displacing anything in the caches.
__device__ __forceinline__ f32x4 ld_state(const f32x4* p) {
  if constexpr (GSA_DECODE_NT) return __builtin_nontemporal_load(p);
  else return *p;
}
__device__ __forceinline__ void st_state(f32x4* p, f32x4 x) {
  if constexpr (GSA_DECODE_NT) __builtin_nontemporal_store(x, p);
  else *p = x;
}

// Threads per unit: KPER float4 of Kt per thread (at most 1024 threads); half
// as many float4 per thread at 128 slots (measured: 1024 threads per unit
// stream 3 % faster there, 512 are best at 64 slots).
template <int DK, int M>
constexpr int decode_threads() {
  constexpr int kper = M >= 128 && GSA_DECODE_KPER > 1 ? GSA_DECODE_KPER / 2 : GSA_DECODE_KPER;
  return (M * DK / 4) / kper > 1024 ? 1024 : (M * DK / 4) / kper;
}

template <typename T, int DK, int DV, int M, int NTH, int ACT>
__global__ void __launch_bounds__(NTH)
gsa_decode_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                  const T* __restrict__ g, float* __restrict__ ks, float* __restrict__ vs,
                  T* __restrict__ o, float inv_tau) {
  constexpr int LK = DK / 4, LV = DV / 4;        // float4 per state row
  constexpr int NK = M * LK / NTH, NV = M * LV / NTH;
  static_assert(NK >= 1 && NV >= 1 && (M * LK) % NTH == 0 && (M * LV) % NTH == 0, "shape");
  static_assert(64 % LK == 0 && 64 % LV == 0, "row width must divide a wave");
  __shared__ float sA[M], sW[M], sZ[M], sS[M];
  __shared__ float sO[NTH / LV][DV];

  const int tid = threadIdx.x;
  const size_t u = blockIdx.x;
  f32x4* kst = reinterpret_cast<f32x4*>(ks + u * M * DK);
  f32x4* vst = reinterpret_cast<f32x4*>(vs + u * M * DV);

  f32x4 kr[NK], vr[NV];
#pragma unroll
  for (int i = 0; i < NK; i++) kr[i] = ld_state(kst + tid + NTH * i);
#pragma unroll
  for (int i = 0; i < NV; i++) vr[i] = ld_state(vst + tid + NTH * i);

  const int ck = tid % LK, cv = tid % LV;       // this thread's float4 column
  float qf[4], kf[4], vf[4];
  load4<T>(q + u * DK + 4 * ck, qf);
  load4<T>(k + u * DK + 4 * ck, kf);
  load4<T>(v + u * DV + 4 * cv, vf);
  for (int c = tid; c < M; c += NTH) {
    float a, w;
    gate_alpha_w(Elem<T>::to_f(g[u * M + c]), inv_tau, a, w);
    sA[c] = a;
    sW[c] = w;
  }
  __syncthreads();

  // pass 1: key state update and slot scores
#pragma unroll
  for (int i = 0; i < NK; i++) {
    const int c = (tid + NTH * i) / LK;
    const float a = sA[c], w = sW[c];
#pragma unroll
    for (int e = 0; e < 4; e++) kr[i][e] = a * kr[i][e] + w * kf[e];
    st_state(kst + tid + NTH * i, kr[i]);
    float z = kr[i][0] * qf[0] + kr[i][1] * qf[1] + kr[i][2] * qf[2] + kr[i][3] * qf[3];
#pragma unroll
    for (int off = LK / 2; off >= 1; off >>= 1) z += __shfl_xor(z, off, 64);
    if (tid % LK == 0) sZ[c] = z;
  }
  __syncthreads();
  if constexpr (ACT != kActSoftmax) {  // element-wise read non-linearity (Table 2 ablations)
    for (int c = tid; c < M; c += NTH) sS[c] = slot_act<ACT>(sZ[c]);
  } else if (tid < 64) {  // slot softmax in wave 0
    float z = -INFINITY;
    for (int c = tid; c < M; c += 64) z = fmaxf(z, sZ[c]);
    float mx = z;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    float sm = 0.f;
    for (int c = tid; c < M; c += 64) sm += __expf(sZ[c] - mx);
    sm = sum64(sm);
    for (int c = tid; c < M; c += 64) sS[c] = __expf(sZ[c] - mx) / sm;
  }
  __syncthreads();

  // pass 2: value state update and read-out
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < NV; i++) {
    const int c = (tid + NTH * i) / LV;
    const float a = sA[c], w = sW[c], s = sS[c];
#pragma unroll
    for (int e = 0; e < 4; e++) {
      vr[i][e] = a * vr[i][e] + w * vf[e];
      acc[e] += s * vr[i][e];
    }
    st_state(vst + tid + NTH * i, vr[i]);
  }
  // threads with the same column: tid % LV equal; rows differ by tid / LV
  const int grp = tid / LV;
#pragma unroll
  for (int e = 0; e < 4; e++) sO[grp][4 * cv + e] = acc[e];
  __syncthreads();
  if (tid < LV) {
    float r[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int gi = 0; gi < NTH / LV; gi++) {
#pragma unroll
      for (int e = 0; e < 4; e++) r[e] += sO[gi][4 * tid + e];
    }
    store4<T>(o + u * DV + 4 * tid, r);
  }
}

template <typename T, int DK, int DV, int M, int ACT>
static int launch_decode(const DecodeLaunch& a) {
  constexpr int NTH = decode_threads<DK, M>();
  const unsigned units = (unsigned)a.N * (unsigned)a.H;
  launch_timed(gsa_decode_kernel<T, DK, DV, M, NTH, ACT>, dim3(units), dim3(NTH), 0, a.stream, a.events, 0,
               1, (const T*)a.q, (const T*)a.k, (const T*)a.v, (const T*)a.g, a.ks, a.vs, (T*)a.o,
               1.0f / a.tau);
  return 0;
}

template <typename T, int DK, int DV, int M>
static int launch_decode_act(const DecodeLaunch& a) {
  switch (a.act) {
    case kActSoftmax: return launch_decode<T, DK, DV, M, kActSoftmax>(a);
    case kActIdentity: return launch_decode<T, DK, DV, M, kActIdentity>(a);
    case kActSwish: return launch_decode<T, DK, DV, M, kActSwish>(a);
    case kActRelu: return launch_decode<T, DK, DV, M, kActRelu>(a);
    case kActRelu2: return launch_decode<T, DK, DV, M, kActRelu2>(a);
    default: return -1;
  }
}

#define DEC_CASE(TT, DTC, DKC, DVC, MC)                                   \
  if (dt == DTC && dk == DKC && dv == DVC && m == MC) {                 \
    if (query) return 1;                                                 \
    return launch_decode_act<TT, DKC, DVC, MC>(*a);                      \
  }

int decode_dispatch(int dt, int dk, int dv, int m, const DecodeLaunch* a, bool query) {
  DEC_CASE(bf16_t, 1, 128, 128, 128)
  DEC_CASE(bf16_t, 1, 128, 128, 64)
  DEC_CASE(bf16_t, 1, 128, 128, 32)
  DEC_CASE(bf16_t, 1, 64, 64, 128)
  DEC_CASE(bf16_t, 1, 64, 64, 64)
  DEC_CASE(bf16_t, 1, 64, 64, 32)
  DEC_CASE(float, 0, 128, 128, 128)
  DEC_CASE(float, 0, 128, 128, 64)
  DEC_CASE(float, 0, 128, 128, 32)
  DEC_CASE(float, 0, 64, 64, 64)
  DEC_CASE(float, 0, 64, 64, 32)
  DEC_CASE(float, 0, 64, 64, 16)
  return -1;
}

// ------------------------------------------------------------- GLA step
// One recurrent GLA step (Sec. 2.3, beta = 1) per (sequence, head), in place:
//   S <- Diag(alpha) S + k v^T,  o = S^T q,  alpha per key dimension (GM: from
// a logit, or a log-decay given directly).  S [dk][dv] fp32 is streamed once:
// thread t owns float4 column c = t % (dv/4) of rows t / (dv/4) + RG j, all its
// rows loaded (non-temporal) before any arithmetic; the partial outputs of
// the RG row groups are summed through LDS.
template <typename T, int DK, int DV, int GM>
__global__ void __launch_bounds__(256)
gla_decode_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                  const T* __restrict__ g, float* __restrict__ ss, T* __restrict__ o, float inv_tau) {
  constexpr int NTH = 256, CPR = DV / 4, RG = NTH / CPR, RPT = DK / RG;
  static_assert(NTH % CPR == 0 && DK % RG == 0 && RPT >= 1, "shape");
  __shared__ float sA[DK], sK[DK], sQ[DK];
  __shared__ float sO[RG][DV];
  const int tid = threadIdx.x;
  const size_t u = blockIdx.x;
  f32x4* st = reinterpret_cast<f32x4*>(ss + u * DK * DV);
  const int c = tid % CPR, r0 = tid / CPR;
  f32x4 sr[RPT];
#pragma unroll
  for (int j = 0; j < RPT; j++) sr[j] = ld_state(st + (size_t)(r0 + RG * j) * CPR + c);
  float vf[4];
  load4<T>(v + u * DV + 4 * c, vf);
  for (int x = tid; x < DK; x += NTH) {
    const float gx = Elem<T>::to_f(g[u * DK + x]);
    sA[x] = GM == kGateLogit ? gate_alpha(gx, inv_tau) : __expf(fminf(gx, 0.f));
    sK[x] = Elem<T>::to_f(k[u * DK + x]);
    sQ[x] = Elem<T>::to_f(q[u * DK + x]);
  }
  __syncthreads();
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < RPT; j++) {
    const int x = r0 + RG * j;
    const float a = sA[x], kx = sK[x], qx = sQ[x];
#pragma unroll
    for (int e = 0; e < 4; e++) {
      sr[j][e] = a * sr[j][e] + kx * vf[e];
      acc[e] += qx * sr[j][e];
    }
    st_state(st + (size_t)x * CPR + c, sr[j]);
  }
#pragma unroll
  for (int e = 0; e < 4; e++) sO[r0][4 * c + e] = acc[e];
  __syncthreads();
  if (tid < CPR) {
    float r[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int gi = 0; gi < RG; gi++) {
#pragma unroll
      for (int e = 0; e < 4; e++) r[e] += sO[gi][4 * tid + e];
    }
    store4<T>(o + u * DV + 4 * tid, r);
  }
}

template <typename T, int DK, int DV>
static int launch_gla_decode(const GlaDecodeLaunch& a) {
  const unsigned units = (unsigned)a.N * (unsigned)a.H;
  const float inv_tau = 1.0f / a.tau;
  if (a.gate_mode == kGateLogit)
    launch_timed(gla_decode_kernel<T, DK, DV, kGateLogit>, dim3(units), dim3(256), 0, a.stream, a.events,
                 0, 1, (const T*)a.q, (const T*)a.k, (const T*)a.v, (const T*)a.g, a.s, (T*)a.o, inv_tau);
  else
    launch_timed(gla_decode_kernel<T, DK, DV, kGateLogDecay>, dim3(units), dim3(256), 0, a.stream,
                 a.events, 0, 1, (const T*)a.q, (const T*)a.k, (const T*)a.v, (const T*)a.g, a.s,
                 (T*)a.o, inv_tau);
  return 0;
}

#define GLA_DEC_CASE(TT, DTC, DKC, DVC)                    \
  if (dt == DTC && dk == DKC && dv == DVC) {               \
    if (query) return 1;                                    \
    return launch_gla_decode<TT, DKC, DVC>(*a);             \
  }

int gla_decode_dispatch(int dt, int dk, int dv, const GlaDecodeLaunch* a, bool query) {
  GLA_DEC_CASE(bf16_t, 1, 128, 128)
  GLA_DEC_CASE(bf16_t, 1, 64, 64)
  GLA_DEC_CASE(float, 0, 128, 128)
  GLA_DEC_CASE(float, 0, 64, 64)
  return -1;
}

__global__ void state_copy_kernel(float* __restrict__ dst, const float* __restrict__ src, size_t n) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) dst[i] = src ? src[i] : 0.f;
}

void record_event(void* const* events, int i, void* stream) {
  if (events && events[i]) (void)hipEventRecord((hipEvent_t)events[i], (hipStream_t)stream);
}

void state_copy(float* dst, const float* src, size_t n, void* stream) {
  if (!dst || n == 0 || dst == src) return;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(state_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, dst, src, n);
}

}  // namespace gsa
