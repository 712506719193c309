// C-ABI boundary of libgsa: argument validation, workspace sizing, dispatch.
// Host code only; every step of the computation runs in the HIP kernels.
#include "../../include/gsa.h"

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include <algorithm>
#include <cmath>

#include "internal.hpp"

namespace {

constexpr int kChunk = 64;
constexpr int kTargetWorkgroups = 256;  // one per CU on MI355X
constexpr int kMaxUnits = 65535;        // grid y limit

bool aligned16(const void* p) { return p == nullptr || ((uintptr_t)p & 15u) == 0; }

struct Range {
  uintptr_t lo, hi;
};
Range rng(const void* p, size_t bytes) { return Range{(uintptr_t)p, (uintptr_t)p + bytes}; }
bool overlap(Range a, Range b) {
  if (a.lo == 0 || b.lo == 0 || a.lo == a.hi || b.lo == b.hi) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

size_t esize(int dtype) { return dtype == GSA_DTYPE_BF16 ? 2 : 4; }

bool dtype_ok(int dtype) { return dtype == GSA_DTYPE_F32 || dtype == GSA_DTYPE_BF16; }

bool nonlinearity_ok(int nl) { return nl >= GSA_SLOT_SOFTMAX && nl <= GSA_SLOT_RELU2; }

int default_chunks_per_seg(long long units, int nchunks) {
  if (nchunks <= 1 || units <= 0) return nchunks > 0 ? nchunks : 1;
  long long p = kTargetWorkgroups / units;
  if (p < 1) p = 1;
  if (p > nchunks) p = nchunks;
  return (int)((nchunks + p - 1) / p);
}

int resolve_cps(long long units, int T, int cps) {
  const int nchunks = (T + kChunk - 1) / kChunk;
  if (cps <= 0) cps = default_chunks_per_seg(units, nchunks);
  if (nchunks > 0 && cps > nchunks) cps = nchunks;
  return cps < 1 ? 1 : cps;
}

// State-map sub-segments per output segment for the bf16 GLA path: enough
// that the state-map pass has about kTargetWorkgroups workgroups (1 for the
// other paths and for single-segment problems).
int gla_state_split(long long units, int T, int cps, int dtype) {
  const int nchunks = (T + kChunk - 1) / kChunk;
  if (dtype != GSA_DTYPE_BF16 || nchunks == 0 || units == 0) return 1;
  const long long P = (nchunks + cps - 1) / cps;
  if (P <= 1) return 1;
  long long r = kTargetWorkgroups / ((P - 1) * units);
  if (r > cps) r = cps;
  return r < 1 ? 1 : (int)r;
}

// Workspace slots per unit: P segment start states, or (P-1) R maps if more.
long long ws_slots(long long P, int R) { return (P - 1) * R > P ? (P - 1) * R : P; }

size_t ws_bytes(long long units, int T, int cps, size_t state_elems, size_t dec_elems, int R = 1) {
  const int nchunks = (T + kChunk - 1) / kChunk;
  if (nchunks == 0 || units == 0) return 0;
  const long long P = (nchunks + cps - 1) / cps;
  if (P <= 1) return 0;
  const long long NQ = ws_slots(P, R);
  const size_t st = (size_t)units * NQ * state_elems * 4;
  const size_t dc = (size_t)units * NQ * dec_elems * 4;
  return ((st + 255) & ~(size_t)255) + dc;
}

// Workspace of a GSA forward over `units` (b, h) units of T tokens (c chunks
// per segment): segment maps and decay products of units * G slot-group units
// (G = slot_groups(dtype, m)), then with G > 1 the groups' output rows
// ([units*T][G][dv], I/O dtype) at *part_off and log-sum-exps ([units*T][G]
// fp32) at *lse_off.
// keep (the training forward): the start states live in the caller's buffer,
// the workspace holds the decay products only (P >= 1 segments).
size_t fwd_ws_bytes(long long units, int T, int c, int dk, int dv, int m, int dtype,
                    size_t* part_off = nullptr, size_t* lse_off = nullptr, bool keep = false) {
  const int G = gsa::slot_groups(dtype, m);
  const int nchunks = (T + kChunk - 1) / kChunk;
  const size_t maps = !keep ? ws_bytes(units * G, T, c, (size_t)(m / G) * (dk + dv), (size_t)(m / G))
                            : (size_t)units * ((nchunks + c - 1) / c) * m * 4;
  if (G == 1 || T == 0 || units == 0) return maps;
  const size_t rows = (size_t)units * T;
  const size_t po = (maps + 255) & ~(size_t)255;
  const size_t lo = (po + rows * G * dv * esize(dtype) + 255) & ~(size_t)255;
  if (part_off) *part_off = po;
  if (lse_off) *lse_off = lo;
  return lo + rows * G * 4;
}

int hip_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? GSA_OK : GSA_ERR_HIP;
}

// A packed variable-length batch: cu (host) holds n + 1 non-decreasing token
// offsets starting at 0.  Also gives the longest length and the chunk count
// over all sequences (one head).
bool varlen_ok(const int* cu, int n, int* tmax, long long* chunks) {
  if (!cu || n < 0 || cu[0] != 0) return false;
  int mx = 0;
  long long ch = 0;
  for (int i = 0; i < n; i++) {
    if (cu[i + 1] < cu[i]) return false;
    const int len = cu[i + 1] - cu[i];
    if (len > mx) mx = len;
    ch += (len + kChunk - 1) / kChunk;
  }
  *tmax = mx;
  *chunks = ch;
  return true;
}

// Chunks per segment for a packed batch: enough segments over all non-empty
// (sequence, head) units for about kTargetWorkgroups output workgroups (equal
// lengths give the dense batch's split).
int resolve_cps_var(int H, int tmax, long long chunks_per_head, int cps) {
  const int nchunks = (tmax + kChunk - 1) / kChunk;
  if (cps <= 0) {
    const long long total = chunks_per_head * H;
    cps = (int)((total + kTargetWorkgroups - 1) / kTargetWorkgroups);
  }
  if (nchunks > 0 && cps > nchunks) cps = nchunks;
  return cps < 1 ? 1 : cps;
}

// Validation of pointers, aliasing and workspace, then the launches; shared by
// the dense batch (cu == nullptr: B sequences of T tokens) and the packed
// variable-length batch (B = n sequences, T = the longest, ntok rows in all).
int gsa_run(const void* q, const void* k, const void* v, const void* g, const float* k0,
            const float* v0, void* o, float* kf, float* vf, int B, int H, int T, size_t ntok, int c,
            const int* cu, int dk, int dv, int m, float tau, int dtype, void* workspace,
            size_t workspace_bytes, int nonlinearity, void* stream, void* const* events,
            float* keep = nullptr, size_t keep_bytes = 0) {
  const long long units = (long long)B * H;
  // units of one launch sequence (a packed batch runs in groups of sequences)
  const long long ws_units = cu ? (long long)std::min(B, gsa::kMaxVarSeqs) * H : units;
  if (ntok > 0 && (!q || !k || !v || !g || !o)) return GSA_ERR_NULL;
  const void* ptrs[] = {q, k, v, g, k0, v0, o, kf, vf, workspace, keep};
  for (const void* p : ptrs)
    if (!aligned16(p)) return GSA_ERR_ALIGN;
  const size_t es = esize(dtype);
  const size_t nt = ntok;
  const Range rq = rng(q, nt * dk * es), rk = rng(k, nt * dk * es), rv = rng(v, nt * dv * es),
              rg = rng(g, nt * m * es), ro = rng(o, nt * dv * es);
  const Range rk0 = rng(k0, (size_t)units * m * dk * 4), rv0 = rng(v0, (size_t)units * m * dv * 4);
  const Range rkf = rng(kf, (size_t)units * m * dk * 4), rvf = rng(vf, (size_t)units * m * dv * 4);
  const Range rws = rng(workspace, workspace_bytes);
  for (Range in : {rq, rk, rv, rg, rk0, rv0, rkf, rvf, rws})
    if (overlap(ro, in)) return GSA_ERR_ALIAS;
  for (Range in : {rq, rk, rv, rg, ro, rws}) {
    if (overlap(rkf, in) || overlap(rvf, in)) return GSA_ERR_ALIAS;
  }
  if (overlap(rkf, rvf) || overlap(rkf, rv0) || overlap(rvf, rk0)) return GSA_ERR_ALIAS;
  if ((kf && k0 && kf != k0 && overlap(rkf, rk0)) || (vf && v0 && vf != v0 && overlap(rvf, rv0)))
    return GSA_ERR_ALIAS;
  for (Range in : {rq, rk, rv, rg, rk0, rv0})
    if (overlap(rws, in)) return GSA_ERR_ALIAS;
  const Range rkeep = rng(keep, keep_bytes);
  for (Range in : {rq, rk, rv, rg, rk0, rv0, ro, rkf, rvf, rws})
    if (overlap(rkeep, in)) return GSA_ERR_ALIAS;
  const int G = gsa::slot_groups(dtype, m);
  if (cu && G > 1) return GSA_ERR_UNSUPPORTED;
  size_t part_off = 0, lse_off = 0;
  const size_t need = fwd_ws_bytes(ws_units, T, c, dk, dv, m, dtype, &part_off, &lse_off, keep != nullptr);
  if (need > 0 && (!workspace || workspace_bytes < need)) return GSA_ERR_WORKSPACE;

  if (T == 0) {  // nothing to read: the final state is the initial state
    gsa::state_copy(kf, k0, (size_t)units * m * dk, stream);
    gsa::state_copy(vf, v0, (size_t)units * m * dv, stream);
    for (int e = 0; e < 4; e++) gsa::record_event(events, e, stream);  // every hook still stamps
    return hip_status();
  }
  gsa::GsaLaunch a{};
  a.q = q; a.k = k; a.v = v; a.g = g; a.k0 = k0; a.v0 = v0; a.o = o; a.kf = kf; a.vf = vf;
  const int nchunks = (T + kChunk - 1) / kChunk;
  const long long P = (nchunks + c - 1) / c;
  if (keep) {
    a.ws_state = keep;
    a.ws_dec = (float*)workspace;
    a.keep_states = keep;
  } else {
    a.ws_state = (float*)workspace;
    a.ws_dec = workspace ? (float*)((char*)workspace +
                                    (((size_t)ws_units * P * m * (dk + dv) * 4 + 255) & ~(size_t)255))
                         : nullptr;
  }
  a.B = B; a.H = H; a.T = T; a.chunks_per_seg = c; a.tau = tau; a.act = nonlinearity;
  a.cu_seqlens = cu; a.n_seqs = cu ? B : 0;
  if (G > 1) {
    a.ws_part = (char*)workspace + part_off;
    a.ws_lse = (float*)((char*)workspace + lse_off);
  }
  a.stream = stream; a.events = events;
  (void)hipGetLastError();
  if (gsa::gsa_dispatch(dtype, dk, dv, m, &a, false) != 0) return GSA_ERR_UNSUPPORTED;
  return hip_status();
}

}  // namespace

extern "C" {

int gsa_abi_version(void) { return GSA_ABI_VERSION; }

const char* gsa_status_string(int s) {
  switch (s) {
    case GSA_OK: return "ok";
    case GSA_ERR_NULL: return "a required pointer is NULL";
    case GSA_ERR_SHAPE: return "invalid size, tau, dtype or non-linearity code";
    case GSA_ERR_ALIGN: return "pointer not 16-byte aligned";
    case GSA_ERR_UNSUPPORTED: return "shape/dtype combination not compiled";
    case GSA_ERR_WORKSPACE: return "workspace missing or too small";
    case GSA_ERR_HIP: return "HIP launch failed";
    case GSA_ERR_ALIAS: return "output overlaps an input or another output";
    case GSA_ERR_SCRATCH_LIMIT: return "problem needs more than the library's fixed scratch";
    default: return "unknown status";
  }
}

int gsa_fwd_supported(int dk, int dv, int m, int C, int dtype) {
  if (C != kChunk || !dtype_ok(dtype)) return 0;
  return gsa::gsa_dispatch(dtype, dk, dv, m, nullptr, true) > 0 ? 1 : 0;
}

int gla_fwd_supported(int dk, int dv, int C, int dtype) {
  if (C != kChunk || !dtype_ok(dtype)) return 0;
  return gsa::gla_dispatch(dtype, dk, dv, nullptr, true) > 0 ? 1 : 0;
}

int gsa_decode_supported(int dk, int dv, int m, int dtype) {
  if (!dtype_ok(dtype)) return 0;
  return gsa::decode_dispatch(dtype, dk, dv, m, nullptr, true) > 0 ? 1 : 0;
}

size_t gsa_fwd_workspace_bytes(int B, int H, int T, int dk, int dv, int m, int C, int dtype,
                               int cps) {
  if (B < 0 || H < 0 || T < 0 || dk < 1 || dv < 1 || m < 1 || C < 1 || !dtype_ok(dtype))
    return (size_t)-1;
  const long long units = (long long)B * H;
  const int G = gsa::slot_groups(dtype, m);
  return fwd_ws_bytes(units, T, resolve_cps(units * G, T, cps), dk, dv, m, dtype);
}

size_t gla_fwd_workspace_bytes(int B, int H, int T, int dk, int dv, int C, int dtype, int cps) {
  if (B < 0 || H < 0 || T < 0 || dk < 1 || dv < 1 || C < 1 || !dtype_ok(dtype)) return (size_t)-1;
  const long long units = (long long)B * H;
  const int c = resolve_cps(units, T, cps);
  return ws_bytes(units, T, c, (size_t)dk * dv, (size_t)dk, gla_state_split(units, T, c, dtype));
}

int gsa_fwd(const void* q, const void* k, const void* v, const void* g, const float* k0,
            const float* v0, void* o, float* kf, float* vf, int B, int H, int T, int dk, int dv, int m,
            int C, float tau, int dtype, void* workspace, size_t workspace_bytes, int cps,
            void* stream) {
  return gsa_fwd_ex(q, k, v, g, k0, v0, o, kf, vf, B, H, T, dk, dv, m, C, tau, dtype, workspace,
                    workspace_bytes, cps, GSA_SLOT_SOFTMAX, stream, nullptr);
}

int gsa_fwd_events(const void* q, const void* k, const void* v, const void* g, const float* k0,
                   const float* v0, void* o, float* kf, float* vf, int B, int H, int T, int dk,
                   int dv, int m, int C, float tau, int dtype, void* workspace,
                   size_t workspace_bytes, int cps, void* stream, void* const* events) {
  return gsa_fwd_ex(q, k, v, g, k0, v0, o, kf, vf, B, H, T, dk, dv, m, C, tau, dtype, workspace,
                    workspace_bytes, cps, GSA_SLOT_SOFTMAX, stream, events);
}

int gsa_fwd_ex(const void* q, const void* k, const void* v, const void* g, const float* k0,
               const float* v0, void* o, float* kf, float* vf, int B, int H, int T, int dk, int dv,
               int m, int C, float tau, int dtype, void* workspace, size_t workspace_bytes, int cps,
               int nonlinearity, void* stream, void* const* events) {
  if (B < 0 || H < 0 || T < 0 || dk < 1 || dv < 1 || m < 1 || C < 1 || !(tau > 0.f) ||
      !std::isfinite(tau) || !dtype_ok(dtype) || !nonlinearity_ok(nonlinearity))
    return GSA_ERR_SHAPE;
  if (!gsa_fwd_supported(dk, dv, m, C, dtype)) return GSA_ERR_UNSUPPORTED;
  const long long units = (long long)B * H;
  const int G = gsa::slot_groups(dtype, m);
  if (units * G > kMaxUnits) return GSA_ERR_UNSUPPORTED;
  if (units == 0) return GSA_OK;
  return gsa_run(q, k, v, g, k0, v0, o, kf, vf, B, H, T, (size_t)units * T,
                 resolve_cps(units * G, T, cps), nullptr, dk, dv, m, tau, dtype, workspace,
                 workspace_bytes, nonlinearity, stream, events);
}

size_t gsa_fwd_varlen_workspace_bytes(const int* cu_seqlens, int n_seqs, int H, int dk, int dv,
                                      int m, int C, int dtype, int cps) {
  int tmax = 0;
  long long total_chunks = 0;
  if (H < 0 || dk < 1 || dv < 1 || m < 1 || C < 1 || !dtype_ok(dtype) ||
      !varlen_ok(cu_seqlens, n_seqs, &tmax, &total_chunks))
    return (size_t)-1;
  const long long ws_units = (long long)std::min(n_seqs, gsa::kMaxVarSeqs) * H;
  return ws_bytes(ws_units, tmax, resolve_cps_var(H, tmax, total_chunks, cps),
                  (size_t)m * (dk + dv), (size_t)m);
}

int gsa_fwd_varlen(const void* q, const void* k, const void* v, const void* g,
                   const int* cu_seqlens, int n_seqs, int H, const float* k0, const float* v0,
                   void* o, float* kf, float* vf, int dk, int dv, int m, int C, float tau, int dtype,
                   void* workspace, size_t workspace_bytes, int cps, void* stream,
                   void* const* events) {
  int tmax = 0;
  long long total_chunks = 0;
  if (H < 0 || dk < 1 || dv < 1 || m < 1 || C < 1 || !(tau > 0.f) || !std::isfinite(tau) ||
      !dtype_ok(dtype) || !varlen_ok(cu_seqlens, n_seqs, &tmax, &total_chunks))
    return GSA_ERR_SHAPE;
  if (dtype != GSA_DTYPE_BF16 || !gsa_fwd_supported(dk, dv, m, C, dtype) || gsa::slot_groups(dtype, m) > 1)
    return GSA_ERR_UNSUPPORTED;
  const long long units = (long long)n_seqs * H;
  if ((long long)std::min(n_seqs, gsa::kMaxVarSeqs) * H > kMaxUnits) return GSA_ERR_UNSUPPORTED;
  if (units == 0) return GSA_OK;
  return gsa_run(q, k, v, g, k0, v0, o, kf, vf, n_seqs, H, tmax,
                 (size_t)H * (size_t)cu_seqlens[n_seqs], resolve_cps_var(H, tmax, total_chunks, cps),
                 cu_seqlens, dk, dv, m, tau, dtype, workspace, workspace_bytes, GSA_SLOT_SOFTMAX,
                 stream, events);
}

int gla_fwd(const void* q, const void* k, const void* v, const void* g, const float* s0, void* o,
            float* sf, int B, int H, int T, int dk, int dv, int C, float tau, int dtype,
            void* workspace, size_t workspace_bytes, int cps, void* stream) {
  return gla_fwd_ex(q, k, v, g, s0, o, sf, B, H, T, dk, dv, C, tau, dtype, workspace,
                    workspace_bytes, cps, GSA_GATE_LOGIT, stream, nullptr);
}

int gla_fwd_events(const void* q, const void* k, const void* v, const void* g, const float* s0,
                   void* o, float* sf, int B, int H, int T, int dk, int dv, int C, float tau,
                   int dtype, void* workspace, size_t workspace_bytes, int cps, void* stream,
                   void* const* events) {
  return gla_fwd_ex(q, k, v, g, s0, o, sf, B, H, T, dk, dv, C, tau, dtype, workspace,
                    workspace_bytes, cps, GSA_GATE_LOGIT, stream, events);
}

int gla_fwd_ex(const void* q, const void* k, const void* v, const void* g, const float* s0, void* o,
               float* sf, int B, int H, int T, int dk, int dv, int C, float tau, int dtype,
               void* workspace, size_t workspace_bytes, int cps, int gate_input, void* stream,
               void* const* events) {
  // tau only scales logits; with log-decays it is not read (any value)
  if (gate_input == GSA_GATE_LOG_DECAY) tau = 1.f;
  if (B < 0 || H < 0 || T < 0 || dk < 1 || dv < 1 || C < 1 || !(tau > 0.f) ||
      !std::isfinite(tau) || !dtype_ok(dtype) ||
      (gate_input != GSA_GATE_LOGIT && gate_input != GSA_GATE_LOG_DECAY))
    return GSA_ERR_SHAPE;
  if (!gla_fwd_supported(dk, dv, C, dtype)) return GSA_ERR_UNSUPPORTED;
  const long long units = (long long)B * H;
  if (units > kMaxUnits) return GSA_ERR_UNSUPPORTED;
  if (units == 0) return GSA_OK;
  if (T > 0 && (!q || !k || !v || !g || !o)) return GSA_ERR_NULL;
  const void* ptrs[] = {q, k, v, g, s0, o, sf, workspace};
  for (const void* p : ptrs)
    if (!aligned16(p)) return GSA_ERR_ALIGN;
  const size_t es = esize(dtype);
  const size_t nt = (size_t)units * T;
  const Range rq = rng(q, nt * dk * es), rk = rng(k, nt * dk * es), rv = rng(v, nt * dv * es),
              rg = rng(g, nt * dk * es), ro = rng(o, nt * dv * es);
  const Range rs0 = rng(s0, (size_t)units * dk * dv * 4), rsf = rng(sf, (size_t)units * dk * dv * 4);
  const Range rws = rng(workspace, workspace_bytes);
  for (Range in : {rq, rk, rv, rg, rs0, rsf, rws})
    if (overlap(ro, in)) return GSA_ERR_ALIAS;
  for (Range in : {rq, rk, rv, rg, rws})
    if (overlap(rsf, in)) return GSA_ERR_ALIAS;
  if (sf && s0 && sf != s0 && overlap(rsf, rs0)) return GSA_ERR_ALIAS;
  for (Range in : {rq, rk, rv, rg, rs0})
    if (overlap(rws, in)) return GSA_ERR_ALIAS;
  const int c = resolve_cps(units, T, cps);
  const int R = gla_state_split(units, T, c, dtype);
  const size_t need = ws_bytes(units, T, c, (size_t)dk * dv, (size_t)dk, R);
  if (need > 0 && (!workspace || workspace_bytes < need)) return GSA_ERR_WORKSPACE;
  if (T == 0) {
    gsa::state_copy(sf, s0, (size_t)units * dk * dv, stream);
    for (int e = 0; e < 4; e++) gsa::record_event(events, e, stream);
    return hip_status();
  }
  gsa::GlaLaunch a{};
  a.q = q; a.k = k; a.v = v; a.g = g; a.s0 = s0; a.o = o; a.sf = sf;
  const int nchunks = (T + kChunk - 1) / kChunk;
  const long long P = (nchunks + c - 1) / c;
  const long long NQ = ws_slots(P, R);
  a.ws_state = (float*)workspace;
  a.ws_dec = workspace ? (float*)((char*)workspace +
                                  (((size_t)units * NQ * dk * dv * 4 + 255) & ~(size_t)255))
                       : nullptr;
  a.B = B; a.H = H; a.T = T; a.chunks_per_seg = c; a.state_split = R; a.tau = tau;
  a.gate_mode = gate_input; a.stream = stream;
  a.events = events;
  (void)hipGetLastError();
  if (gsa::gla_dispatch(dtype, dk, dv, &a, false) != 0) return GSA_ERR_UNSUPPORTED;
  return hip_status();
}

int gsa_decode_step(const void* q, const void* k, const void* v, const void* g, float* ks,
                    float* vs, void* o, int N, int H, int dk, int dv, int m, float tau, int dtype,
                    void* stream) {
  return gsa_decode_step_ex(q, k, v, g, ks, vs, o, N, H, dk, dv, m, tau, dtype, GSA_SLOT_SOFTMAX,
                            stream, nullptr);
}

int gsa_decode_step_events(const void* q, const void* k, const void* v, const void* g, float* ks,
                           float* vs, void* o, int N, int H, int dk, int dv, int m, float tau,
                           int dtype, void* stream, void* const* events) {
  return gsa_decode_step_ex(q, k, v, g, ks, vs, o, N, H, dk, dv, m, tau, dtype, GSA_SLOT_SOFTMAX,
                            stream, events);
}

int gsa_decode_step_ex(const void* q, const void* k, const void* v, const void* g, float* ks,
                       float* vs, void* o, int N, int H, int dk, int dv, int m, float tau, int dtype,
                       int nonlinearity, void* stream, void* const* events) {
  if (N < 0 || H < 0 || dk < 1 || dv < 1 || m < 1 || !(tau > 0.f) || !std::isfinite(tau) ||
      !dtype_ok(dtype) || !nonlinearity_ok(nonlinearity))
    return GSA_ERR_SHAPE;
  if (!gsa_decode_supported(dk, dv, m, dtype)) return GSA_ERR_UNSUPPORTED;
  const long long units = (long long)N * H;
  if (units == 0) return GSA_OK;
  if (units > 0x7fffffffLL) return GSA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !g || !ks || !vs || !o) return GSA_ERR_NULL;
  const void* ptrs[] = {q, k, v, g, ks, vs, o};
  for (const void* p : ptrs)
    if (!aligned16(p)) return GSA_ERR_ALIGN;
  const size_t es = esize(dtype);
  const Range rq = rng(q, units * dk * es), rk = rng(k, units * dk * es), rv = rng(v, units * dv * es),
              rg = rng(g, units * m * es), ro = rng(o, units * dv * es);
  const Range rks = rng(ks, (size_t)units * m * dk * 4), rvs = rng(vs, (size_t)units * m * dv * 4);
  if (overlap(rks, rvs)) return GSA_ERR_ALIAS;
  for (Range in : {rq, rk, rv, rg, ro}) {
    if (overlap(rks, in) || overlap(rvs, in)) return GSA_ERR_ALIAS;
  }
  for (Range in : {rq, rk, rv, rg})
    if (overlap(ro, in)) return GSA_ERR_ALIAS;
  gsa::DecodeLaunch a{};
  a.q = q; a.k = k; a.v = v; a.g = g; a.ks = ks; a.vs = vs; a.o = o; a.N = N; a.H = H;
  a.tau = tau; a.act = nonlinearity; a.stream = stream; a.events = events;
  (void)hipGetLastError();
  if (gsa::decode_dispatch(dtype, dk, dv, m, &a, false) != 0) return GSA_ERR_UNSUPPORTED;
  return hip_status();
}

int gla_decode_supported(int dk, int dv, int dtype) {
  if (!dtype_ok(dtype)) return 0;
  return gsa::gla_decode_dispatch(dtype, dk, dv, nullptr, true) > 0 ? 1 : 0;
}

int gla_decode_step(const void* q, const void* k, const void* v, const void* g, float* s, void* o,
                    int N, int H, int dk, int dv, float tau, int dtype, int gate_input, void* stream,
                    void* const* events) {
  if (gate_input == GSA_GATE_LOG_DECAY) tau = 1.f;  // not read
  if (N < 0 || H < 0 || dk < 1 || dv < 1 || !(tau > 0.f) || !std::isfinite(tau) ||
      !dtype_ok(dtype) || (gate_input != GSA_GATE_LOGIT && gate_input != GSA_GATE_LOG_DECAY))
    return GSA_ERR_SHAPE;
  if (!gla_decode_supported(dk, dv, dtype)) return GSA_ERR_UNSUPPORTED;
  const long long units = (long long)N * H;
  if (units == 0) return GSA_OK;
  if (units > 0x7fffffffLL) return GSA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !g || !s || !o) return GSA_ERR_NULL;
  const void* ptrs[] = {q, k, v, g, s, o};
  for (const void* p : ptrs)
    if (!aligned16(p)) return GSA_ERR_ALIGN;
  const size_t es = esize(dtype);
  const Range rq = rng(q, units * dk * es), rk = rng(k, units * dk * es), rv = rng(v, units * dv * es),
              rg = rng(g, units * dk * es), ro = rng(o, units * dv * es);
  const Range rs = rng(s, (size_t)units * dk * dv * 4);
  for (Range in : {rq, rk, rv, rg, ro})
    if (overlap(rs, in)) return GSA_ERR_ALIAS;
  for (Range in : {rq, rk, rv, rg})
    if (overlap(ro, in)) return GSA_ERR_ALIAS;
  gsa::GlaDecodeLaunch a{};
  a.q = q; a.k = k; a.v = v; a.g = g; a.s = s; a.o = o; a.N = N; a.H = H; a.tau = tau;
  a.gate_mode = gate_input; a.stream = stream; a.events = events;
  (void)hipGetLastError();
  if (gsa::gla_decode_dispatch(dtype, dk, dv, &a, false) != 0) return GSA_ERR_UNSUPPORTED;
  return hip_status();
}

size_t gsa_bwd_workspace_bytes_ex(int B, int H, int T, int dk, int dv, int m, int dtype, int nonlinearity) {
  if (B < 0 || H < 0 || T < 0 || dk < 1 || dv < 1 || m < 1 || !dtype_ok(dtype) ||
      !nonlinearity_ok(nonlinearity))
    return 0;
  if (T == 0) return 0;
  const size_t units = (size_t)B * H;
  return gsa::gsa_bwd_need_bytes(dtype, nonlinearity, false, units, ((size_t)T + kChunk - 1) / kChunk,
                                 units * T, T, dk, dv, m);
}

size_t gsa_bwd_workspace_bytes(int B, int H, int T, int dk, int dv, int m) {
  // enough for either storage type and any read (the token-walk path's need
  // is the larger)
  return std::max(gsa_bwd_workspace_bytes_ex(B, H, T, dk, dv, m, GSA_DTYPE_F32, GSA_SLOT_SOFTMAX),
                  gsa_bwd_workspace_bytes_ex(B, H, T, dk, dv, m, GSA_DTYPE_BF16, GSA_SLOT_SOFTMAX));
}

size_t gsa_bwd_varlen_workspace_bytes(const int* cu_seqlens, int n_seqs, int H, int dk, int dv, int m) {
  int tmax = 0;
  long long chunks = 0;
  if (H < 0 || dk < 1 || dv < 1 || m < 1 || !varlen_ok(cu_seqlens, n_seqs, &tmax, &chunks)) return 0;
  return gsa::gsa_bwd_ws_bytes((size_t)std::min(n_seqs, gsa::kMaxVarSeqs) * H,
                               ((size_t)tmax + kChunk - 1) / kChunk,
                               (size_t)H * (size_t)cu_seqlens[n_seqs], dk, dv, m);
}

int gsa_bwd_supported(int dk, int dv, int m, int dtype) {
  if (!dtype_ok(dtype)) return 0;
  return gsa::gsa_bwd_dispatch(dtype, dk, dv, m, nullptr, true) == 0;
}

// Validation and launch shared by the dense batch (cu == nullptr: B sequences
// of T tokens) and the packed variable-length batch (B = n sequences, T = the
// longest, ntok rows in all).
static int bwd_run(const void* q, const void* k, const void* v, const void* g, const void* d_o,
                   const float* k0, const float* v0, const float* d_kf, const float* d_vf, void* d_q,
                   void* d_k, void* d_v, void* d_g, float* d_k0, float* d_v0, int B, int H, int T,
                   size_t ntok, const int* cu, int dk, int dv, int m, float tau, int dtype,
                   void* workspace, size_t workspace_bytes, int nonlinearity, void* stream,
                   void* const* events, const float* saved = nullptr, size_t saved_bytes = 0) {
  if (!gsa_bwd_supported(dk, dv, m, dtype)) return GSA_ERR_UNSUPPORTED;
  if (saved && !gsa::gsa_bwd_on_mfma(dtype, nonlinearity, cu != nullptr)) return GSA_ERR_UNSUPPORTED;
  // two slot groups (bf16, m = 128): dense batches and the smooth reads only
  if (gsa::slot_groups(dtype, m) > 1 && (cu || nonlinearity == GSA_SLOT_RELU)) return GSA_ERR_UNSUPPORTED;
  const long long units = (long long)B * H;
  if (units == 0) return GSA_OK;
  // one grid row per unit of a launch sequence (a packed batch launches groups)
  const long long launch_units = cu ? (long long)std::min(B, gsa::kMaxVarSeqs) * H : units;
  // 128 slots run as two groups of 64, each group a unit of the launches
  if (launch_units * gsa::slot_groups(dtype, m) > 65535) return GSA_ERR_UNSUPPORTED;
  if (((long long)T + kChunk - 1) / kChunk > 65535) return GSA_ERR_UNSUPPORTED;  // chunks: grid y
  if (ntok > 0 && (!q || !k || !v || !g || !d_o || !d_q || !d_k || !d_v || !d_g))
    return GSA_ERR_NULL;
  const void* ptrs[] = {q, k, v, g, d_o, k0, v0, d_kf, d_vf, d_q, d_k, d_v, d_g, d_k0, d_v0, workspace, saved};
  for (const void* p : ptrs)
    if (!aligned16(p)) return GSA_ERR_ALIGN;
  const size_t es = esize(dtype);
  const size_t sk = (size_t)units * m * dk * 4, sv = (size_t)units * m * dv * 4;
  const Range rq = rng(q, ntok * dk * es), rk = rng(k, ntok * dk * es), rv = rng(v, ntok * dv * es),
              rg = rng(g, ntok * m * es), rdo = rng(d_o, ntok * dv * es);
  const Range rk0 = rng(k0, sk), rv0 = rng(v0, sv), rkf = rng(d_kf, sk), rvf = rng(d_vf, sv);
  const Range rdq = rng(d_q, ntok * dk * es), rdk = rng(d_k, ntok * dk * es),
              rdv = rng(d_v, ntok * dv * es), rdg = rng(d_g, ntok * m * es);
  const Range rdk0 = rng(d_k0, sk), rdv0 = rng(d_v0, sv);
  const size_t need = T > 0 ? gsa::gsa_bwd_need_bytes(dtype, nonlinearity, cu != nullptr, (size_t)launch_units,
                                                      ((size_t)T + kChunk - 1) / kChunk, ntok, T, dk, dv, m)
                            : 0;
  const Range rws = rng(workspace, need);
  const Range outs[] = {rdq, rdk, rdv, rdg, rdk0, rdv0, rws};
  const Range rsaved = rng(saved, saved_bytes);
  for (Range out : outs)
    if (overlap(out, rsaved)) return GSA_ERR_ALIAS;
  const Range ins[] = {rq, rk, rv, rg, rdo, rk0, rv0, rkf, rvf};
  for (int i = 0; i < 7; i++) {
    for (Range in : ins)
      if (overlap(outs[i], in)) return GSA_ERR_ALIAS;
    for (int j = i + 1; j < 7; j++)
      if (overlap(outs[i], outs[j])) return GSA_ERR_ALIAS;
  }
  if (need > 0 && (!workspace || workspace_bytes < need)) return GSA_ERR_WORKSPACE;
  gsa::GsaBwdLaunch a{};
  a.q = q; a.k = k; a.v = v; a.g = g; a.d_o = d_o;
  a.k0 = k0; a.v0 = v0; a.dkf = d_kf; a.dvf = d_vf;
  a.dq = d_q; a.dk = d_k; a.dv = d_v; a.dg = d_g; a.dk0 = d_k0; a.dv0 = d_v0;
  a.ws = (float*)workspace;
  a.B = B; a.H = H; a.T = T; a.tau = tau; a.act = nonlinearity;
  a.cu_seqlens = cu; a.n_seqs = cu ? B : 0;
  a.saved_states = saved;
  a.stream = stream; a.events = events;
  (void)hipGetLastError();
  if (gsa::gsa_bwd_dispatch(dtype, dk, dv, m, &a, false) != 0) return GSA_ERR_UNSUPPORTED;
  return hip_status();
}

int gsa_bwd_ex(const void* q, const void* k, const void* v, const void* g, const void* d_o,
               const float* k0, const float* v0, const float* d_kf, const float* d_vf, void* d_q,
               void* d_k, void* d_v, void* d_g, float* d_k0, float* d_v0, int B, int H, int T,
               int dk, int dv, int m, float tau, int dtype, void* workspace, size_t workspace_bytes,
               int nonlinearity, void* stream, void* const* events) {
  if (B < 0 || H < 0 || T < 0 || dk < 1 || dv < 1 || m < 1 || !(tau > 0.f) ||
      !std::isfinite(tau) || !dtype_ok(dtype) || !nonlinearity_ok(nonlinearity))
    return GSA_ERR_SHAPE;
  return bwd_run(q, k, v, g, d_o, k0, v0, d_kf, d_vf, d_q, d_k, d_v, d_g, d_k0, d_v0, B, H, T,
                 (size_t)B * H * T, nullptr, dk, dv, m, tau, dtype, workspace, workspace_bytes,
                 nonlinearity, stream, events);
}

int gsa_bwd_varlen(const void* q, const void* k, const void* v, const void* g, const void* d_o,
                   const int* cu_seqlens, int n_seqs, int H, const float* k0, const float* v0,
                   const float* d_kf, const float* d_vf, void* d_q, void* d_k, void* d_v, void* d_g,
                   float* d_k0, float* d_v0, int dk, int dv, int m, float tau, int dtype,
                   void* workspace, size_t workspace_bytes, void* stream, void* const* events) {
  int tmax = 0;
  long long chunks = 0;
  if (H < 0 || dk < 1 || dv < 1 || m < 1 || !(tau > 0.f) || !std::isfinite(tau) ||
      !dtype_ok(dtype) || !varlen_ok(cu_seqlens, n_seqs, &tmax, &chunks))
    return GSA_ERR_SHAPE;
  return bwd_run(q, k, v, g, d_o, k0, v0, d_kf, d_vf, d_q, d_k, d_v, d_g, d_k0, d_v0, n_seqs, H, tmax,
                 (size_t)H * (size_t)cu_seqlens[n_seqs], cu_seqlens, dk, dv, m, tau, dtype, workspace,
                 workspace_bytes, GSA_SLOT_SOFTMAX, stream, events);
}

// ---------------------------------------------------------------- training pair
// The chunks per segment of the training pair: the matrix-core backward's split
// of this problem (units * groups units).
static int train_cps(long long units, int T, int G) {
  return gsa::gsa_bwd_chunks_per_segment(units * G, (T + kChunk - 1) / kChunk);
}

// The pair runs where the backward runs on the matrix cores: bf16, every read
// but ReLU (dense batches only, checked by the entry points).
static bool train_ok(int dk, int dv, int m, int dtype, int nonlinearity) {
  return dtype == GSA_DTYPE_BF16 && gsa_fwd_supported(dk, dv, m, kChunk, dtype) &&
         gsa_bwd_supported(dk, dv, m, dtype) && gsa::gsa_bwd_on_mfma(dtype, nonlinearity, false);
}

size_t gsa_train_states_bytes(int B, int H, int T, int dk, int dv, int m, int dtype) {
  if (B < 0 || H < 0 || T < 0 || dk < 1 || dv < 1 || m < 1 || !dtype_ok(dtype)) return (size_t)-1;
  if (!train_ok(dk, dv, m, dtype, GSA_SLOT_SOFTMAX) || T == 0) return 0;
  const long long units = (long long)B * H;
  const int G = gsa::slot_groups(dtype, m), c = train_cps(units, T, G);
  const long long P = ((T + kChunk - 1) / kChunk + c - 1) / c;
  return (size_t)units * P * m * (dk + dv) * 4;
}

size_t gsa_fwd_train_workspace_bytes(int B, int H, int T, int dk, int dv, int m, int dtype) {
  if (B < 0 || H < 0 || T < 0 || dk < 1 || dv < 1 || m < 1 || !dtype_ok(dtype)) return (size_t)-1;
  const long long units = (long long)B * H;
  const int G = gsa::slot_groups(dtype, m);
  return fwd_ws_bytes(units, T, train_cps(units, T, G), dk, dv, m, dtype, nullptr, nullptr, true);
}

int gsa_fwd_train(const void* q, const void* k, const void* v, const void* g, const float* k0,
                  const float* v0, void* o, float* kf, float* vf, int B, int H, int T, int dk, int dv,
                  int m, float tau, int dtype, void* workspace, size_t workspace_bytes,
                  float* states, size_t states_bytes, int nonlinearity, void* stream,
                  void* const* events) {
  if (B < 0 || H < 0 || T < 0 || dk < 1 || dv < 1 || m < 1 || !(tau > 0.f) || !std::isfinite(tau) ||
      !dtype_ok(dtype) || !nonlinearity_ok(nonlinearity))
    return GSA_ERR_SHAPE;
  if (!train_ok(dk, dv, m, dtype, nonlinearity)) return GSA_ERR_UNSUPPORTED;
  const long long units = (long long)B * H;
  const int G = gsa::slot_groups(dtype, m);
  if (units * G > kMaxUnits) return GSA_ERR_UNSUPPORTED;
  if (units == 0) return GSA_OK;
  const size_t need = gsa_train_states_bytes(B, H, T, dk, dv, m, dtype);
  if (need > 0 && !states) return GSA_ERR_NULL;
  if (states_bytes < need) return GSA_ERR_WORKSPACE;
  return gsa_run(q, k, v, g, k0, v0, o, kf, vf, B, H, T, (size_t)units * T, train_cps(units, T, G),
                 nullptr, dk, dv, m, tau, dtype, workspace, workspace_bytes, nonlinearity, stream, events,
                 need > 0 ? states : nullptr, need);
}

int gsa_bwd_train(const void* q, const void* k, const void* v, const void* g, const void* d_o,
                  const float* k0, const float* v0, const float* d_kf, const float* d_vf, void* d_q,
                  void* d_k, void* d_v, void* d_g, float* d_k0, float* d_v0, int B, int H, int T,
                  int dk, int dv, int m, float tau, int dtype, void* workspace, size_t workspace_bytes,
                  const float* states, size_t states_bytes, int nonlinearity, void* stream,
                  void* const* events) {
  if (B < 0 || H < 0 || T < 0 || dk < 1 || dv < 1 || m < 1 || !(tau > 0.f) ||
      !std::isfinite(tau) || !dtype_ok(dtype) || !nonlinearity_ok(nonlinearity))
    return GSA_ERR_SHAPE;
  if (!train_ok(dk, dv, m, dtype, nonlinearity)) return GSA_ERR_UNSUPPORTED;
  const size_t need = gsa_train_states_bytes(B, H, T, dk, dv, m, dtype);
  if (need > 0 && !states) return GSA_ERR_NULL;
  if (states_bytes < need) return GSA_ERR_WORKSPACE;
  return bwd_run(q, k, v, g, d_o, k0, v0, d_kf, d_vf, d_q, d_k, d_v, d_g, d_k0, d_v0, B, H, T,
                 (size_t)B * H * T, nullptr, dk, dv, m, tau, dtype, workspace, workspace_bytes,
                 nonlinearity, stream, events, need > 0 ? states : nullptr, need);
}

int gsa_bwd(const void* q, const void* k, const void* v, const void* g, const void* d_o,
            const float* k0, const float* v0, const float* d_kf, const float* d_vf, void* d_q,
            void* d_k, void* d_v, void* d_g, float* d_k0, float* d_v0, int B, int H, int T,
            int dk, int dv, int m, float tau, int dtype, void* workspace, size_t workspace_bytes,
            void* stream, void* const* events) {
  return gsa_bwd_ex(q, k, v, g, d_o, k0, v0, d_kf, d_vf, d_q, d_k, d_v, d_g, d_k0, d_v0, B, H, T,
                    dk, dv, m, tau, dtype, workspace, workspace_bytes, GSA_SLOT_SOFTMAX, stream,
                    events);
}

}  // extern "C"
