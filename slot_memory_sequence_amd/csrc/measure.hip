// Calibration kernels: what this GPU actually sustains, measured beside the
// published peaks (HBM3E 8 TB/s, dense bf16 MFMA 2.5 PFLOP/s).  Not part of the
// method; the benchmark reports the GSA kernels against both figures.
//
//  * gsa_measure_hbm: a streaming copy, or an in-place update, float4
//    non-temporal loads and stores, one contiguous 32 KB block per workgroup
//    with all of a thread's loads in flight before its stores (bytes moved =
//    2 x size).
//  * gsa_measure_mfma_bf16: a register-only loop of v_mfma_f32_16x16x32_bf16
//    with eight independent accumulator chains per wave, four waves per SIMD
//    on every CU; no memory traffic in the loop.  With all-ones operands every
//    accumulator element gains 32 per iteration, so the result is checkable.
#include "../../include/gsa.h"
#include "common.hpp"
#include "internal.hpp"
#include "launch.hpp"

namespace gsa {
namespace {

constexpr int kCopyThreads = 256;
constexpr int kCopyPer = 8;               // float4 per thread: 32 KB per workgroup
constexpr int kMfmaThreads = 256;         // four waves
constexpr int kMfmaChains = 8;            // independent accumulators per wave

// Each workgroup streams one contiguous 32 KB block: every thread issues its
// eight loads (each a fully coalesced 4 KB row of the block) before any
// store.  UPDATE = 0 copies src to dst; UPDATE = 1 adds 1 to dst in place
// (src unused), the read-modify-write pattern of the decode kernel's states.
// (A sweep of block shapes on this GPU: 256 threads x 8 float4 streamed best,
// 6.1 TB/s copy and 5.9 TB/s update on 1 GiB, against 5.1-5.5 with 16 per
// thread and 5.3-5.5 with 1024-thread workgroups.)
template <int UPDATE>
__global__ void __launch_bounds__(kCopyThreads)
hbm_stream_kernel(const f32x4* __restrict__ src, f32x4* __restrict__ dst, size_t n4) {
  const f32x4* in = UPDATE ? dst : src;
  const size_t base = (size_t)blockIdx.x * (kCopyThreads * kCopyPer) + threadIdx.x;
  f32x4 r[kCopyPer];
  if (base + (size_t)(kCopyPer - 1) * kCopyThreads < n4) {
#pragma unroll
    for (int j = 0; j < kCopyPer; j++) r[j] = __builtin_nontemporal_load(in + base + j * kCopyThreads);
#pragma unroll
    for (int j = 0; j < kCopyPer; j++) {
      if (UPDATE) r[j] += 1.f;
      __builtin_nontemporal_store(r[j], dst + base + j * kCopyThreads);
    }
  } else {
    for (int j = 0; j < kCopyPer; j++) {
      const size_t i = base + (size_t)j * kCopyThreads;
      if (i < n4) {
        f32x4 x = __builtin_nontemporal_load(in + i);
        if (UPDATE) x += 1.f;
        __builtin_nontemporal_store(x, dst + i);
      }
    }
  }
}

// one = 1.0 in every operand element (passed in, so the compiler cannot fold
// the loop); the sink gets one value per workgroup: the sum over the
// workgroup's first lane of every accumulator element, 1024 * iters + 496
__global__ void __launch_bounds__(kMfmaThreads)
mfma_bf16_kernel(float* __restrict__ sink, int iters, float one) {
  bf16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; j++) {
    a[j] = (__bf16)one;
    b[j] = (__bf16)one;
  }
  // distinct starting values, so that no two chains are the same computation
  f32x4 c[kMfmaChains];
#pragma unroll
  for (int k = 0; k < kMfmaChains; k++)
    c[k] = f32x4{(4 * k) * one, (4 * k + 1) * one, (4 * k + 2) * one, (4 * k + 3) * one};
  for (int i = 0; i < iters; i++) {
#pragma unroll
    for (int k = 0; k < kMfmaChains; k++) c[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[k], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < kMfmaChains; k++) s += c[k][0] + c[k][1] + c[k][2] + c[k][3];
  if (threadIdx.x == 0) sink[blockIdx.x] = s;
}

}  // namespace
}  // namespace gsa

extern "C" {

int gsa_measure_hbm(const void* src, void* dst, size_t bytes, int mode, void* stream,
                    void* const* events) {
  if (mode != 0 && mode != 1) return GSA_ERR_SHAPE;
  if (!dst || (mode == 0 && !src)) return GSA_ERR_NULL;
  if (bytes == 0 || bytes % 16 != 0) return GSA_ERR_SHAPE;
  if (((uintptr_t)src & 15u) || ((uintptr_t)dst & 15u)) return GSA_ERR_ALIGN;
  const uintptr_t s0 = (uintptr_t)src, d0 = (uintptr_t)dst;
  if (mode == 0 && s0 < d0 + bytes && d0 < s0 + bytes) return GSA_ERR_ALIAS;
  const size_t n4 = bytes / 16, per_block = (size_t)gsa::kCopyThreads * gsa::kCopyPer;
  const size_t blocks = (n4 + per_block - 1) / per_block;
  if (blocks > 0x7fffffffu) return GSA_ERR_SHAPE;
  (void)hipGetLastError();
  if (mode == 0)
    gsa::launch_timed(gsa::hbm_stream_kernel<0>, dim3((unsigned)blocks), dim3(gsa::kCopyThreads), 0,
                      stream, events, 0, 1, (const gsa::f32x4*)src, (gsa::f32x4*)dst, n4);
  else
    gsa::launch_timed(gsa::hbm_stream_kernel<1>, dim3((unsigned)blocks), dim3(gsa::kCopyThreads), 0,
                      stream, events, 0, 1, (const gsa::f32x4*)src, (gsa::f32x4*)dst, n4);
  return hipGetLastError() == hipSuccess ? GSA_OK : GSA_ERR_HIP;
}

int gsa_measure_mfma_bf16(float* sink, size_t sink_floats, int iterations, double* flops,
                          void* stream, void* const* events) {
  if (!sink) return GSA_ERR_NULL;
  if (iterations < 1) return GSA_ERR_SHAPE;
  if (sink_floats < GSA_MEASURE_MFMA_WORKGROUPS) return GSA_ERR_WORKSPACE;
  if ((uintptr_t)sink & 15u) return GSA_ERR_ALIGN;
  (void)hipGetLastError();
  gsa::launch_timed(gsa::mfma_bf16_kernel, dim3(GSA_MEASURE_MFMA_WORKGROUPS), dim3(gsa::kMfmaThreads),
                    0, stream, events, 0, 1, sink, iterations, 1.0f);
  if (flops)
    *flops = (double)GSA_MEASURE_MFMA_WORKGROUPS * (gsa::kMfmaThreads / 64) * (double)iterations *
             gsa::kMfmaChains * (2.0 * 16 * 16 * 32);
  return hipGetLastError() == hipSuccess ? GSA_OK : GSA_ERR_HIP;
}

}  // extern "C"
