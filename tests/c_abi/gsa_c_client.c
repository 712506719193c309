/*
 * A plain C client of libgsa: no Python, no PyTorch.  It allocates device
 * buffers with the HIP runtime, calls gsa_fwd, gsa_bwd on the same inputs and
 * gsa_decode_step on the forward's final states through include/gsa.h, and
 * writes the results to a file, so that a test can compare them with the fp64
 * oracle on the same inputs.
 *
 * Then the same inputs once more in bfloat16 storage (the inputs are chosen
 * exactly representable there): the training pair gsa_fwd_train /
 * gsa_bwd_train on the matrix-core path, and gsa_fwd_noalloc, which takes no
 * workspace at all.
 *
 * Usage: gsa_c_client <in.bin> <out.bin>
 *   in.bin : int32 B, H, T, dk, dv, m; then float32 q[B,H,T,dk], k[B,H,T,dk],
 *            v[B,H,T,dv], g[B,H,T,m], and one decode token per unit:
 *            q1[B,H,dk], k1[B,H,dk], v1[B,H,dv], g1[B,H,m]; then the output
 *            gradient d_o[B,H,T,dv]
 *   out.bin: float32 o[B,H,T,dv], k_final[B,H,m,dk], v_final[B,H,m,dv],
 *            o1[B,H,dv], the states after the decode step, and the
 *            gradients d_q, d_k [B,H,T,dk], d_v [B,H,T,dv], d_g [B,H,T,m];
 *            then from the bf16 calls, widened to float32: the training
 *            forward's o, k_final, v_final, the pair's d_q, d_k, d_v, d_g,
 *            and the no-allocation forward's o.
 * Exit status 0 on success; any library or runtime error is printed.
 */
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/gsa.h"

#define HIP_OK(x)                                                               \
  do {                                                                          \
    hipError_t e_ = (x);                                                        \
    if (e_ != hipSuccess) {                                                     \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));           \
      return 2;                                                                 \
    }                                                                           \
  } while (0)

static float* read_floats(FILE* f, size_t n) {
  float* p = (float*)malloc(n * sizeof(float) + 1);
  if (p && fread(p, sizeof(float), n, f) != n) {
    free(p);
    return NULL;
  }
  return p;
}

/* float32 -> bfloat16 bits, rounding to nearest even (the inputs here are
   already representable, so this is exact) */
static unsigned short to_bf16(float x) {
  unsigned int u;
  memcpy(&u, &x, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (unsigned short)(u >> 16);
}
static float from_bf16(unsigned short b) {
  unsigned int u = (unsigned int)b << 16;
  float x;
  memcpy(&x, &u, 4);
  return x;
}
static int to_device_bf16(unsigned short** d, const float* h, size_t n) {
  unsigned short* t = (unsigned short*)malloc(n * 2 + 2);
  if (!t) return 1;
  for (size_t i = 0; i < n; i++) t[i] = to_bf16(h[i]);
  int bad = hipMalloc((void**)d, n * 2 + 16) != hipSuccess ||
            (n && hipMemcpy(*d, t, n * 2, hipMemcpyHostToDevice) != hipSuccess);
  free(t);
  return bad;
}

static int to_device(float** d, const float* h, size_t n) {
  if (hipMalloc((void**)d, n * sizeof(float) + 16) != hipSuccess) return 1;
  if (n && hipMemcpy(*d, h, n * sizeof(float), hipMemcpyHostToDevice) != hipSuccess) return 1;
  return 0;
}

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s in.bin out.bin\n", argv[0]);
    return 1;
  }
  FILE* fi = fopen(argv[1], "rb");
  if (!fi) return 1;
  int hdr[6];
  if (fread(hdr, sizeof(int), 6, fi) != 6) return 1;
  const int B = hdr[0], H = hdr[1], T = hdr[2], dk = hdr[3], dv = hdr[4], m = hdr[5];
  const size_t U = (size_t)B * H;
  const size_t nq = U * T * dk, nv = U * T * dv, ng = U * T * m;
  float* hq = read_floats(fi, nq);
  float* hk = read_floats(fi, nq);
  float* hv = read_floats(fi, nv);
  float* hg = read_floats(fi, ng);
  float* hq1 = read_floats(fi, U * dk);
  float* hk1 = read_floats(fi, U * dk);
  float* hv1 = read_floats(fi, U * dv);
  float* hg1 = read_floats(fi, U * m);
  float* hdo = read_floats(fi, nv);
  fclose(fi);
  if (!hq || !hk || !hv || !hg || !hq1 || !hk1 || !hv1 || !hg1 || !hdo) {
    fprintf(stderr, "short input file\n");
    return 1;
  }
  if (gsa_abi_version() != GSA_ABI_VERSION) {
    fprintf(stderr, "ABI version mismatch: library %d, header %d\n", gsa_abi_version(),
            GSA_ABI_VERSION);
    return 1;
  }
  if (!gsa_fwd_supported(dk, dv, m, 64, GSA_DTYPE_F32) || !gsa_bwd_supported(dk, dv, m, GSA_DTYPE_F32)) {
    fprintf(stderr, "shape not compiled\n");
    return 1;
  }

  float *q, *k, *v, *g, *o, *kf, *vf, *q1, *k1, *v1, *g1, *o1, *d_o, *gq, *gk, *gv, *gg;
  if (to_device(&q, hq, nq) || to_device(&k, hk, nq) || to_device(&v, hv, nv) ||
      to_device(&g, hg, ng) || to_device(&q1, hq1, U * dk) || to_device(&k1, hk1, U * dk) ||
      to_device(&v1, hv1, U * dv) || to_device(&g1, hg1, U * m) || to_device(&d_o, hdo, nv)) {
    fprintf(stderr, "device allocation or copy failed\n");
    return 2;
  }
  HIP_OK(hipMalloc((void**)&o, nv * sizeof(float) + 16));
  HIP_OK(hipMalloc((void**)&kf, U * m * dk * sizeof(float)));
  HIP_OK(hipMalloc((void**)&vf, U * m * dv * sizeof(float)));
  HIP_OK(hipMalloc((void**)&o1, U * dv * sizeof(float)));
  HIP_OK(hipMalloc((void**)&gq, nq * sizeof(float) + 16));
  HIP_OK(hipMalloc((void**)&gk, nq * sizeof(float) + 16));
  HIP_OK(hipMalloc((void**)&gv, nv * sizeof(float) + 16));
  HIP_OK(hipMalloc((void**)&gg, ng * sizeof(float) + 16));

  hipStream_t st;
  HIP_OK(hipStreamCreate(&st));
  const size_t wsb = gsa_fwd_workspace_bytes(B, H, T, dk, dv, m, 64, GSA_DTYPE_F32, 0);
  void* ws = NULL;
  if (wsb == (size_t)-1) return 1;
  if (wsb) HIP_OK(hipMalloc(&ws, wsb));

  int s = gsa_fwd(q, k, v, g, NULL, NULL, o, kf, vf, B, H, T, dk, dv, m, 64, 8.0f, GSA_DTYPE_F32,
                  ws, wsb, 0, st);
  if (s != GSA_OK) {
    fprintf(stderr, "gsa_fwd: %s\n", gsa_status_string(s));
    return 3;
  }
  /* an error is reported on the host before anything runs */
  if (gsa_fwd(q, k, v, g, NULL, NULL, o, kf, vf, B, H, T, dk, dv, m, 64, -1.0f, GSA_DTYPE_F32, ws,
              wsb, 0, st) != GSA_ERR_SHAPE) {
    fprintf(stderr, "bad tau was not rejected\n");
    return 3;
  }
  HIP_OK(hipStreamSynchronize(st));

  FILE* fo = fopen(argv[2], "wb");
  if (!fo) return 1;
  size_t nbuf = nv > U * m * (dk + dv) ? nv : U * m * (dk + dv);
  if (nq > nbuf) nbuf = nq;
  if (ng > nbuf) nbuf = ng;
  float* buf = (float*)malloc(nbuf * sizeof(float));
  if (!buf) return 1;
#define DUMP(dptr, n)                                                            \
  do {                                                                           \
    HIP_OK(hipMemcpy(buf, dptr, (n) * sizeof(float), hipMemcpyDeviceToHost));   \
    if (fwrite(buf, sizeof(float), (n), fo) != (n)) return 1;                    \
  } while (0)
  DUMP(o, nv);
  DUMP(kf, U * m * dk);
  DUMP(vf, U * m * dv);

  /* the backward of the same forward (zero initial states, no final-state
     gradients), with a workspace of its own */
  const size_t wsb2 = gsa_bwd_workspace_bytes(B, H, T, dk, dv, m);
  void* ws2 = NULL;
  if (wsb2) HIP_OK(hipMalloc(&ws2, wsb2));
  s = gsa_bwd(q, k, v, g, d_o, NULL, NULL, NULL, NULL, gq, gk, gv, gg, NULL, NULL, B, H, T, dk, dv,
              m, 8.0f, GSA_DTYPE_F32, ws2, wsb2, st, NULL);
  if (s != GSA_OK) {
    fprintf(stderr, "gsa_bwd: %s\n", gsa_status_string(s));
    return 3;
  }
  if (gsa_bwd(q, k, v, g, d_o, NULL, NULL, NULL, NULL, gq, gk, gv, gg, NULL, NULL, B, H, T, dk, dv,
              m, 8.0f, GSA_DTYPE_F32, ws2, wsb2 - 16, st, NULL) != GSA_ERR_WORKSPACE) {
    fprintf(stderr, "short backward workspace was not rejected\n");
    return 3;
  }

  /* one decode step from the final states, in place */
  s = gsa_decode_step(q1, k1, v1, g1, kf, vf, o1, B, H, dk, dv, m, 8.0f, GSA_DTYPE_F32, st);
  if (s != GSA_OK) {
    fprintf(stderr, "gsa_decode_step: %s\n", gsa_status_string(s));
    return 3;
  }
  HIP_OK(hipStreamSynchronize(st));
  DUMP(o1, U * dv);
  DUMP(kf, U * m * dk);
  DUMP(vf, U * m * dv);
  DUMP(gq, nq);
  DUMP(gk, nq);
  DUMP(gv, nv);
  DUMP(gg, ng);

  /* ---- bf16 storage: the training pair and the no-allocation forward */
  if (!gsa_fwd_supported(dk, dv, m, 64, GSA_DTYPE_BF16) || !gsa_bwd_supported(dk, dv, m, GSA_DTYPE_BF16)) {
    fprintf(stderr, "bf16 shape not compiled\n");
    return 1;
  }
  unsigned short *bq, *bk, *bv, *bg, *bdo, *bo, *bo2, *bgq, *bgk, *bgv, *bgg;
  if (to_device_bf16(&bq, hq, nq) || to_device_bf16(&bk, hk, nq) || to_device_bf16(&bv, hv, nv) ||
      to_device_bf16(&bg, hg, ng) || to_device_bf16(&bdo, hdo, nv)) {
    fprintf(stderr, "device allocation or copy failed\n");
    return 2;
  }
  HIP_OK(hipMalloc((void**)&bo, nv * 2 + 16));
  HIP_OK(hipMalloc((void**)&bo2, nv * 2 + 16));
  HIP_OK(hipMalloc((void**)&bgq, nq * 2 + 16));
  HIP_OK(hipMalloc((void**)&bgk, nq * 2 + 16));
  HIP_OK(hipMalloc((void**)&bgv, nv * 2 + 16));
  HIP_OK(hipMalloc((void**)&bgg, ng * 2 + 16));
  const size_t stb = gsa_train_states_bytes(B, H, T, dk, dv, m, GSA_DTYPE_BF16);
  const size_t fwb = gsa_fwd_train_workspace_bytes(B, H, T, dk, dv, m, GSA_DTYPE_BF16);
  const size_t bwb = gsa_bwd_workspace_bytes_ex(B, H, T, dk, dv, m, GSA_DTYPE_BF16, GSA_SLOT_SOFTMAX);
  if (stb == (size_t)-1 || fwb == (size_t)-1) return 1;
  float* states = NULL;
  void *fws = NULL, *bws = NULL;
  if (stb) HIP_OK(hipMalloc((void**)&states, stb));
  if (fwb) HIP_OK(hipMalloc(&fws, fwb));
  if (bwb) HIP_OK(hipMalloc(&bws, bwb));
  s = gsa_fwd_train(bq, bk, bv, bg, NULL, NULL, bo, kf, vf, B, H, T, dk, dv, m, 8.0f, GSA_DTYPE_BF16,
                    fws, fwb, states, stb, GSA_SLOT_SOFTMAX, st, NULL);
  if (s != GSA_OK) {
    fprintf(stderr, "gsa_fwd_train: %s\n", gsa_status_string(s));
    return 3;
  }
  s = gsa_bwd_train(bq, bk, bv, bg, bdo, NULL, NULL, NULL, NULL, bgq, bgk, bgv, bgg, NULL, NULL, B, H, T,
                    dk, dv, m, 8.0f, GSA_DTYPE_BF16, bws, bwb, states, stb, GSA_SLOT_SOFTMAX, st, NULL);
  if (s != GSA_OK) {
    fprintf(stderr, "gsa_bwd_train: %s\n", gsa_status_string(s));
    return 3;
  }
  s = gsa_fwd_noalloc(bq, bk, bv, bg, NULL, NULL, bo2, NULL, NULL, B, H, T, dk, dv, m, 64, 8.0f,
                      GSA_DTYPE_BF16, 0, GSA_SLOT_SOFTMAX, st, NULL);
  if (s != GSA_OK) {
    fprintf(stderr, "gsa_fwd_noalloc: %s\n", gsa_status_string(s));
    return 3;
  }
  HIP_OK(hipStreamSynchronize(st));
  unsigned short* hb = (unsigned short*)malloc(nbuf * 2);
  if (!hb) return 1;
#define DUMP_BF16(dptr, n)                                                       \
  do {                                                                           \
    HIP_OK(hipMemcpy(hb, dptr, (n) * 2, hipMemcpyDeviceToHost));                \
    for (size_t i_ = 0; i_ < (n); i_++) buf[i_] = from_bf16(hb[i_]);           \
    if (fwrite(buf, sizeof(float), (n), fo) != (n)) return 1;                    \
  } while (0)
  DUMP_BF16(bo, nv);
  DUMP(kf, U * m * dk);
  DUMP(vf, U * m * dv);
  DUMP_BF16(bgq, nq);
  DUMP_BF16(bgk, nq);
  DUMP_BF16(bgv, nv);
  DUMP_BF16(bgg, ng);
  DUMP_BF16(bo2, nv);
  fclose(fo);
  printf("gsa_c_client ok: B=%d H=%d T=%d dk=%d dv=%d m=%d workspace=%zu\n", B, H, T, dk, dv, m, wsb);
  return 0;
}
