// The C-ABI layer's host code (argument validation, aliasing checks,
// workspace sizing, launch descriptors) under AddressSanitizer and
// UndefinedBehaviorSanitizer, with the kernel dispatchers replaced by stubs
// that record the launch descriptor instead of launching.  No GPU and no HIP
// runtime are involved: every pointer below is a fake device address that
// nothing dereferences.  Exit status 0 when every check passes.
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>

#include "../../include/gsa.h"
#include "../../slot_memory_sequence_amd/csrc/internal.hpp"

// ------------------------------------------------------------ stubs
static int g_launches = 0;
static gsa::GsaLaunch g_gsa;
static gsa::GsaBwdLaunch g_bwd;

static bool shape_ok(int dk, int dv, int m) {
  return dk == dv && (dk == 64 || dk == 128) && m >= 16 && m <= 128 && (m & (m - 1)) == 0;
}
extern "C" hipError_t hipGetLastError(void) { return hipSuccess; }
namespace gsa {
int gsa_dispatch(int, int dk, int dv, int m, const GsaLaunch* a, bool query) {
  if (!shape_ok(dk, dv, m)) return -1;
  if (query) return 1;
  g_gsa = *a;
  g_launches++;
  return 0;
}
int gla_dispatch(int, int dk, int dv, const GlaLaunch*, bool query) {
  if (!shape_ok(dk, dv, 64)) return -1;
  if (!query) g_launches++;
  return query ? 1 : 0;
}
int decode_dispatch(int, int dk, int dv, int m, const DecodeLaunch*, bool query) {
  if (!shape_ok(dk, dv, m)) return -1;
  if (!query) g_launches++;
  return query ? 1 : 0;
}
int gla_decode_dispatch(int, int dk, int dv, const GlaDecodeLaunch*, bool query) {
  if (!shape_ok(dk, dv, 64)) return -1;
  if (!query) g_launches++;
  return query ? 1 : 0;
}
int gsa_bwd_dispatch(int, int dk, int dv, int m, const GsaBwdLaunch* a, bool query) {
  if (!shape_ok(dk, dv, m)) return -1;
  if (query) return 0;
  g_bwd = *a;
  g_launches++;
  return 0;
}
size_t gsa_bwd_ws_bytes(size_t units, size_t chunks, size_t rows, int dk, int dv, int m) {
  return (units * chunks * (size_t)m * (dk + dv) + rows * (size_t)m) * 4;
}
size_t gsa_bwd_need_bytes(int dtype, int act, bool packed, size_t units, size_t chunks, size_t rows, int T,
                          int dk, int dv, int m) {
  return gsa_bwd_ws_bytes(units, chunks, rows, dk, dv, m) / (gsa_bwd_on_mfma(dtype, act, packed) ? 2 : 1) +
         (size_t)T * 0;
}
int gsa_bwd_chunks_per_segment(long long units, int nchunks) {
  const long long p = units > 0 && units < 256 ? 256 / units : 1;
  const long long s = (nchunks + p - 1) / p;
  return (int)(s < 1 ? 1 : s > 8 ? 8 : s);
}
void state_copy(float*, const float*, size_t, void*) {}
void record_event(void* const*, int, void*) {}
}  // namespace gsa

// ------------------------------------------------------------ driver
static int fails = 0;
#define CHECK(cond)                                                  \
  do {                                                               \
    if (!(cond)) {                                                   \
      printf("FAIL line %d: %s\n", __LINE__, #cond);                 \
      fails++;                                                       \
    }                                                                \
  } while (0)

static void* A(uintptr_t x) { return (void*)x; }
static const uintptr_t MB = 1 << 20;

int main() {
  // fake, disjoint, 16-byte-aligned device ranges
  void *q = A(1 * 256 * MB), *k = A(2 * 256 * MB), *v = A(3 * 256 * MB), *g = A(4 * 256 * MB);
  void* o = A(5 * 256 * MB);
  float* st = (float*)A(6 * 256 * MB);
  float* fin = (float*)A(7 * 256 * MB);
  void* ws = A(8 * 256 * MB);
  const int B = 8, H = 4, T = 2048, d = 128, m = 64;
  // ---- gsa_fwd: accepted calls reach the dispatcher with a carved workspace
  size_t nb = gsa_fwd_workspace_bytes(B, H, T, d, d, m, 64, GSA_DTYPE_BF16, 0);
  CHECK(nb > 0 && nb != (size_t)-1);
  int r = gsa_fwd(q, k, v, g, st, st + B * H * m * d, o, fin, fin + B * H * m * d, B, H, T, d, d, m,
                  64, 8.f, GSA_DTYPE_BF16, ws, nb, 0, nullptr);
  CHECK(r == GSA_OK && g_launches == 1);
  CHECK((uintptr_t)g_gsa.ws_state == (uintptr_t)ws);
  CHECK((uintptr_t)g_gsa.ws_dec > (uintptr_t)ws && (uintptr_t)g_gsa.ws_dec < (uintptr_t)ws + nb);
  CHECK(g_gsa.chunks_per_seg >= 1);
  // ---- rejections, nothing dispatched
  const int before = g_launches;
  CHECK(gsa_fwd(q, k, v, g, nullptr, nullptr, o, nullptr, nullptr, B, H, T, d, d, m, 64, 8.f,
                GSA_DTYPE_BF16, ws, nb - 1, 0, nullptr) == GSA_ERR_WORKSPACE);
  CHECK(gsa_fwd(q, k, v, g, nullptr, nullptr, q, nullptr, nullptr, B, H, T, d, d, m, 64, 8.f,
                GSA_DTYPE_BF16, ws, nb, 0, nullptr) == GSA_ERR_ALIAS);
  CHECK(gsa_fwd(q, k, v, g, nullptr, nullptr, (char*)o + 8, nullptr, nullptr, B, H, T, d, d, m, 64,
                8.f, GSA_DTYPE_BF16, ws, nb, 0, nullptr) == GSA_ERR_ALIGN);
  CHECK(gsa_fwd(nullptr, k, v, g, nullptr, nullptr, o, nullptr, nullptr, B, H, T, d, d, m, 64, 8.f,
                GSA_DTYPE_BF16, ws, nb, 0, nullptr) == GSA_ERR_NULL);
  CHECK(gsa_fwd(q, k, v, g, nullptr, nullptr, o, nullptr, nullptr, B, H, T, d, d, m, 64, -1.f,
                GSA_DTYPE_BF16, ws, nb, 0, nullptr) == GSA_ERR_SHAPE);
  CHECK(gsa_fwd(q, k, v, g, nullptr, nullptr, o, nullptr, nullptr, B, H, T, 96, 96, m, 64, 8.f,
                GSA_DTYPE_BF16, ws, nb, 0, nullptr) == GSA_ERR_UNSUPPORTED);
  CHECK(gsa_fwd(q, k, v, g, nullptr, nullptr, o, nullptr, nullptr, 70000, 1, T, d, d, m, 64, 8.f,
                GSA_DTYPE_BF16, ws, (size_t)-1, 0, nullptr) == GSA_ERR_UNSUPPORTED);
  CHECK(gsa_fwd(q, k, v, g, nullptr, nullptr, o, ws == nullptr ? nullptr : (float*)ws, nullptr, B, H,
                T, d, d, m, 64, 8.f, GSA_DTYPE_BF16, ws, nb, 0, nullptr) == GSA_ERR_ALIAS);
  CHECK(g_launches == before);
  // T = 0 and empty batches: nothing to launch
  CHECK(gsa_fwd(nullptr, nullptr, nullptr, nullptr, st, nullptr, nullptr, fin, nullptr, 2, 2, 0, d, d,
                m, 64, 8.f, GSA_DTYPE_F32, nullptr, 0, 0, nullptr) == GSA_OK);
  CHECK(gsa_fwd_workspace_bytes(0, 4, 100, d, d, m, 64, 1, 0) == 0);
  CHECK(gsa_fwd_workspace_bytes(1, 1, 1 << 30, d, d, m, 64, 1, 1) != (size_t)-1);
  // ---- packed batches: offsets validated on the host
  const int cu_ok[] = {0, 100, 100, 900, 901};
  const int cu_bad[] = {0, 100, 50, 900, 901};
  size_t nv = gsa_fwd_varlen_workspace_bytes(cu_ok, 4, H, d, d, m, 64, 1, 0);
  CHECK(nv != (size_t)-1);
  CHECK(gsa_fwd_varlen(q, k, v, g, cu_ok, 4, H, nullptr, nullptr, o, fin, nullptr, d, d, m, 64, 8.f,
                       GSA_DTYPE_BF16, ws, nv, 0, nullptr, nullptr) == GSA_OK);
  CHECK(g_gsa.cu_seqlens == cu_ok && g_gsa.n_seqs == 4);
  CHECK(gsa_fwd_varlen(q, k, v, g, cu_bad, 4, H, nullptr, nullptr, o, nullptr, nullptr, d, d, m, 64,
                       8.f, GSA_DTYPE_BF16, ws, nv, 0, nullptr, nullptr) == GSA_ERR_SHAPE);
  CHECK(gsa_fwd_varlen_workspace_bytes(cu_bad, 4, H, d, d, m, 64, 1, 0) == (size_t)-1);
  CHECK(gsa_fwd_varlen_workspace_bytes(nullptr, 4, H, d, d, m, 64, 1, 0) == (size_t)-1);
  // ---- GLA and the decode steps
  size_t ng = gla_fwd_workspace_bytes(8, 16, 4096, d, d, 64, 1, 0);
  CHECK(gla_fwd(q, k, v, g, nullptr, o, nullptr, 8, 16, 4096, d, d, 64, 16.f, 1, ws, ng, 0, nullptr) ==
        GSA_OK);
  CHECK(gla_fwd(q, k, v, g, nullptr, o, nullptr, 8, 16, 4096, d, d, 64, 16.f, 1, ws, ng / 2, 0,
                nullptr) == GSA_ERR_WORKSPACE);
  CHECK(gla_fwd_ex(q, k, v, g, nullptr, o, nullptr, 8, 16, 4096, d, d, 64, 0.f, 1, ws, ng, 0, 7,
                   nullptr, nullptr) == GSA_ERR_SHAPE);
  CHECK(gsa_decode_step(q, k, v, g, st, fin, o, 256, 16, d, d, m, 8.f, 1, nullptr) == GSA_OK);
  CHECK(gsa_decode_step(q, k, v, g, st, st + 16, o, 256, 16, d, d, m, 8.f, 1, nullptr) ==
        GSA_ERR_ALIAS);
  CHECK(gsa_decode_step_ex(q, k, v, g, st, fin, o, 256, 16, d, d, m, 8.f, 1, 9, nullptr, nullptr) ==
        GSA_ERR_SHAPE);
  CHECK(gla_decode_step(q, k, v, g, st, o, 256, 16, d, d, 16.f, 1, 0, nullptr, nullptr) == GSA_OK);
  CHECK(gla_decode_step(q, k, v, g, (float*)o, o, 256, 16, d, d, 16.f, 1, 0, nullptr, nullptr) ==
        GSA_ERR_ALIAS);
  // ---- backward
  void *dq = A(9 * 256 * MB), *dk = A(10 * 256 * MB), *dv = A(11 * 256 * MB), *dg = A(12 * 256 * MB);
  void* dO = A(13 * 256 * MB);
  size_t nbw = gsa_bwd_workspace_bytes_ex(B, H, T, d, d, m, GSA_DTYPE_BF16, GSA_SLOT_SOFTMAX);
  CHECK(nbw > 0 && nbw < gsa_bwd_workspace_bytes(B, H, T, d, d, m));
  CHECK(gsa_bwd(q, k, v, g, dO, nullptr, nullptr, nullptr, nullptr, dq, dk, dv, dg, nullptr, nullptr, B,
                H, T, d, d, m, 8.f, 1, ws, nbw, nullptr, nullptr) == GSA_OK);
  CHECK(g_bwd.ws == (float*)ws && g_bwd.T == T);
  CHECK(gsa_bwd(q, k, v, g, dO, nullptr, nullptr, nullptr, nullptr, dq, dk, dv, dg, nullptr, nullptr, B,
                H, T, d, d, m, 8.f, 1, ws, nbw - 4, nullptr, nullptr) == GSA_ERR_WORKSPACE);
  CHECK(gsa_bwd(q, k, v, g, dO, nullptr, nullptr, nullptr, nullptr, dq, dq, dv, dg, nullptr, nullptr, B,
                H, T, d, d, m, 8.f, 1, ws, nbw, nullptr, nullptr) == GSA_ERR_ALIAS);
  CHECK(gsa_bwd_ex(q, k, v, g, dO, nullptr, nullptr, nullptr, nullptr, dq, dk, dv, dg, nullptr, nullptr,
                   B, H, T, d, d, m, 8.f, 1, ws, nbw, 5, nullptr, nullptr) == GSA_ERR_SHAPE);
  size_t nbv = gsa_bwd_varlen_workspace_bytes(cu_ok, 4, H, d, d, m);
  CHECK(gsa_bwd_varlen(q, k, v, g, dO, cu_ok, 4, H, nullptr, nullptr, nullptr, nullptr, dq, dk, dv, dg,
                       nullptr, nullptr, d, d, m, 8.f, 1, ws, nbv, nullptr, nullptr) == GSA_OK);
  CHECK(gsa_bwd_varlen(q, k, v, g, dO, cu_bad, 4, H, nullptr, nullptr, nullptr, nullptr, dq, dk, dv, dg,
                       nullptr, nullptr, d, d, m, 8.f, 1, ws, nbv, nullptr, nullptr) == GSA_ERR_SHAPE);
  for (int s = -1; s < 9; s++) CHECK(gsa_status_string(s) != nullptr);
  printf("%s (%d launches recorded)\n", fails ? "FAILED" : "all ok", g_launches);
  return fails ? 1 : 0;
}
