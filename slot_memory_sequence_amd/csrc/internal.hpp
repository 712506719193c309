// Internal launch descriptors shared by the C-ABI layer and the kernel files.
#pragma once
#include <stddef.h>

namespace gsa {

constexpr int kLdsBytes = 160 * 1024;  // LDS per workgroup on gfx950
constexpr int kMaxVarSeqs = 256;       // sequences per launch of a variable-length batch

struct GsaLaunch {
  const void *q, *k, *v, *g;
  const float *k0, *v0;
  void* o;
  float *kf, *vf;
  float *ws_state, *ws_dec;
  int B, H, T, chunks_per_seg;
  float tau;
  int act;  // slot read non-linearity, a GSA_SLOT_* code (SlotAct)
  // Packed variable-length batch (bf16 only): n_seqs sequences, host offsets
  // cu_seqlens[0..n_seqs] (validated), T = the longest length, B = n_seqs;
  // launched in groups of at most kMaxVarSeqs sequences, whose workspace is
  // sized for min(n_seqs, kMaxVarSeqs) * H units.
  // cu_seqlens == nullptr: the dense [B, H, T, d] batch.
  const int* cu_seqlens;
  int n_seqs;
  // two slot groups (slot_groups(dtype, m) == 2, dense batches only): the
  // groups' output rows [B*H*T][2][dv] (I/O dtype) and log-sum-exps
  // [B*H*T][2] fp32, in the workspace after the segment maps
  void* ws_part;
  float* ws_lse;
  // nullable: keep the segment start states for the backward.  ws_state is
  // then this buffer ([units * groups][P][m / groups][dk+dv] fp32), the maps
  // are never folded by the output kernel, and the scan also runs for P = 1
  // (its one slot is the initial state).
  float* keep_states;
  void* stream;
  void* const* events;  // nullable: 4 hipEvent_t, see gsa_fwd_events
};

// Slot groups a GSA call with m slots runs as: 2 for bf16 at m = 128 (two
// groups of 64 merged by the read's log-sum-exp), else 1.
inline int slot_groups(int dtype, int m) { return dtype == 1 && m == 128 ? 2 : 1; }

struct GlaLaunch {
  const void *q, *k, *v, *g;
  const float* s0;
  void* o;
  float* sf;
  float *ws_state, *ws_dec;
  int B, H, T, chunks_per_seg;
  int state_split;  // bf16: state-map sub-segments per output segment (>= 1)
  float tau;
  int gate_mode;  // how g is given: a GSA_GATE_* code (GateMode)
  void* stream;
  void* const* events;  // nullable: 4 hipEvent_t, see gla_fwd_events
};

// record events[i] on the stream when the event array and entry are non-null
void record_event(void* const* events, int i, void* stream);

struct DecodeLaunch {
  const void *q, *k, *v, *g;
  float *ks, *vs;
  void* o;
  int N, H;
  float tau;
  int act;  // slot read non-linearity, a GSA_SLOT_* code (SlotAct)
  void* stream;
  void* const* events;  // nullable: 2 hipEvent_t, start and end of the kernel
};

struct GlaDecodeLaunch {
  const void *q, *k, *v, *g;
  float* s;
  void* o;
  int N, H;
  float tau;
  int gate_mode;  // a GSA_GATE_* code (GateMode)
  void* stream;
  void* const* events;  // nullable: 2 hipEvent_t, start and end of the kernel
};

// query == true: return the phase-C LDS bytes (> 0) if the shape is compiled, else -1.
// query == false: enqueue the launches and return 0, or -1 if not compiled.
int gsa_dispatch(int dtype, int dk, int dv, int m, const GsaLaunch* a, bool query);
int gsa_dispatch_bf16(int dk, int dv, int m, const GsaLaunch* a, bool query);
int gla_dispatch(int dtype, int dk, int dv, const GlaLaunch* a, bool query);
int gla_dispatch_bf16(int dk, int dv, const GlaLaunch* a, bool query);
int decode_dispatch(int dtype, int dk, int dv, int m, const DecodeLaunch* a, bool query);
int gla_decode_dispatch(int dtype, int dk, int dv, const GlaDecodeLaunch* a, bool query);
// copy (src != null) or zero-fill n floats on the stream (T == 0 state hand-off)
void state_copy(float* dst, const float* src, size_t n, void* stream);

// GSA backward: gradients of q, k, v, g (I/O dtype) and of the initial states
// (fp32, nullable), given d_o and the nullable final-state gradients dkf / dvf.
struct GsaBwdLaunch {
  const void *q, *k, *v, *g, *d_o;
  const float *k0, *v0, *dkf, *dvf;
  void *dq, *dk, *dv, *dg;
  float *dk0, *dv0;
  float* ws;
  int B, H, T;
  float tau;
  int act;  // slot read non-linearity, a GSA_SLOT_* code (SlotAct)
  // packed variable-length batch (nullable): host offsets cu_seqlens[0..n_seqs]
  // (validated), B = n_seqs, T = the longest length, rows [H, total, d]
  const int* cu_seqlens;
  int n_seqs;
  // nullable: the segment start states a training forward kept (the
  // matrix-core path reads them instead of recomputing them)
  const float* saved_states;
  void* stream;
  void* const* events;  // nullable: 4 hipEvent_t around the two token-walk kernels
};
// The bf16 forward's segment start states of a dense batch (state maps of
// segments 0 .. P-2, then the per-unit scan): ws_state [units][P][m][dk+dv]
// fp32, slot p = the state at the start of segment p (S chunks each); ws_dec
// [units][P][m] fp32.  groups = 2: the units are the slot groups of m = 64
// each of a batch with 128 slots (unit 2u + h, gate row pitch 128).  Returns
// -1 if (dk, dv, m, groups) is not compiled.
int gsa_bf16_segment_states(int dk, int dv, int m, int groups, const void* k, const void* v, const void* g,
                            const float* k0, const float* v0, float* ws_state, float* ws_dec,
                            int units, int T, int S, int P, float tau, void* stream);

// workspace of one launch sequence of `units` units of `chunks` chunks over
// `rows` token rows in all
size_t gsa_bwd_ws_bytes(size_t units, size_t chunks, size_t rows, int dk, int dv, int m);
int gsa_bwd_dispatch(int dtype, int dk, int dv, int m, const GsaBwdLaunch* a, bool query);
// The dense bf16 backward on the matrix cores (the chunk form): query ->
// workspace bytes for `units` units of T tokens; launch -> 0; -1 if (dk, dv,
// m) is not compiled for it.
long long gsa_bwd_bf16_dispatch(int dk, int dv, int m, const GsaBwdLaunch* a, bool query, size_t units, int T);
// Chunks per segment of the matrix-core backward for `units` (group) units of
// nchunks chunks: the split a training forward keeps its start states for.
int gsa_bwd_chunks_per_segment(long long units, int nchunks);
// Workspace bytes of the backward a call with these arguments runs: the
// matrix-core path for a dense bf16 batch, the token-walk path otherwise
// (float32, packed batches: `rows` token rows, `units` units of `chunks`
// chunks per launch sequence).
size_t gsa_bwd_need_bytes(int dtype, int act, bool packed, size_t units, size_t chunks, size_t rows, int T,
                          int dk, int dv, int m);
// Whether a call runs the matrix-core backward: dense bf16 batches of every
// read but ReLU, whose derivative is a step at z = 0 -- there the token walk's
// fp32 scores keep the step on the same side as the exact z, bf16 operands do not.
inline bool gsa_bwd_on_mfma(int dtype, int act, bool packed) { return dtype == 1 && !packed && act != 3; }

}  // namespace gsa
