/* A plain C caller of the Kamera C ABI (include/kamera.h), with no Python or torch:
 * one GQA chunk (2 KV heads x 128, bf16, 2 layers) is rehydrated at a new position
 * with rank-8 factors on K and V (Kamera preprint Eq. 1: KV = R(delta) KV_stored + U V^T)
 * into dense output rows.
 *
 *   rehydrate_demo IN OUT T DELTA [noalloc]
 *
 * With "noalloc" the call is kamera_rehydrate_batched_noalloc (no workspace, no allocation)
 * instead of kamera_rehydrate_batched with a hipMalloc'd workspace.
 *
 * IN holds, as raw little-endian bf16 bit patterns, in this order: K [2][T][256],
 * V [2][T][256], U_K [2][T][8], V_K [2][256][8], U_V [2][T][8], V_V [2][256][8].
 * OUT receives K_out [2][T][256] then V_out [2][T][256]. Exit status 0 on success; any
 * failed call prints the library's status and detail and exits with status 1. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kamera.h"

enum { LAYERS = 2, HEADS = 2, HEAD_DIM = 128, F = HEADS * HEAD_DIM, RANK = 8 };

static int hip_ok(hipError_t e, const char* what) {
  if (e == hipSuccess) return 1;
  fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
  return 0;
}

static int kamera_ok(kamera_status st, const char* what) {
  if (st == KAMERA_OK) return 1;
  fprintf(stderr, "%s: %s (%s)\n", what, kamera_status_string(st), kamera_last_error());
  return 0;
}

int main(int argc, char** argv) {
  if (argc != 5 && !(argc == 6 && strcmp(argv[5], "noalloc") == 0)) {
    fprintf(stderr, "usage: %s IN OUT T DELTA [noalloc]\n", argv[0]);
    return 2;
  }
  const int noalloc = argc == 6;
  const int64_t T = atoll(argv[3]);
  const int64_t delta = atoll(argv[4]);
  if (T < 1 || T > (1 << 20)) return 2;
  const size_t rows = (size_t)LAYERS * T * F, urows = (size_t)LAYERS * T * RANK, vrows = (size_t)LAYERS * F * RANK;
  const size_t n_in = 2 * rows + 2 * (urows + vrows);
  uint16_t* host = (uint16_t*)malloc(n_in * sizeof(uint16_t));
  uint16_t* out = (uint16_t*)malloc(2 * rows * sizeof(uint16_t));
  if (!host || !out) return 1;
  FILE* f = fopen(argv[1], "rb");
  if (!f || fread(host, sizeof(uint16_t), n_in, f) != n_in) {
    fprintf(stderr, "cannot read %zu values from %s\n", n_in, argv[1]);
    return 1;
  }
  fclose(f);

  uint16_t* dev = NULL;  /* inputs, then the two outputs */
  if (!hip_ok(hipMalloc((void**)&dev, (n_in + 2 * rows) * sizeof(uint16_t)), "hipMalloc")) return 1;
  if (!hip_ok(hipMemcpy(dev, host, n_in * sizeof(uint16_t), hipMemcpyHostToDevice), "hipMemcpy")) return 1;
  uint16_t *k = dev, *v = k + rows, *uk = v + rows, *vk = uk + urows, *uv = vk + vrows, *vv = uv + urows;
  uint16_t *k_out = vv + vrows, *v_out = k_out + rows;

  kamera_layout lay;
  memset(&lay, 0, sizeof(lay));
  lay.family = KAMERA_GQA;
  lay.dtype = KAMERA_BF16;
  lay.num_layers = LAYERS;
  lay.num_kv_heads = HEADS;
  lay.head_dim = HEAD_DIM;
  lay.pairing = KAMERA_NEOX;
  lay.page_size = 16;
  lay.rope_base = 1e6;

  kamera_chunk c;
  memset(&c, 0, sizeof(c));
  c.num_tokens = (int32_t)T;
  c.flags = KAMERA_PATCH;
  c.delta = delta;
  c.k_src = k;
  c.v_src = v;
  c.k_dst = k_out;
  c.v_dst = v_out;
  c.num_factors = 2;
  c.factors[0].u = uk;
  c.factors[0].v = vk;
  c.factors[0].tensor = 0;
  c.factors[0].width = F;
  c.factors[0].rank = RANK;
  c.factors[1] = c.factors[0];
  c.factors[1].u = uv;
  c.factors[1].v = vv;
  c.factors[1].tensor = 1;

  void* ws = NULL;
  if (noalloc) {
    if (!kamera_ok(kamera_rehydrate_batched_noalloc(&lay, &c, 1, NULL, NULL), "kamera_rehydrate_batched_noalloc"))
      return 1;
  } else {
    const size_t ws_bytes = kamera_batch_workspace_bytes(&lay, &c, 1);
    if (ws_bytes == 0 || !hip_ok(hipMalloc(&ws, ws_bytes), "hipMalloc(workspace)")) return 1;
    if (!kamera_ok(kamera_rehydrate_batched(&lay, &c, 1, NULL, ws, ws_bytes, NULL), "kamera_rehydrate_batched"))
      return 1;
  }
  if (!hip_ok(hipDeviceSynchronize(), "hipDeviceSynchronize")) return 1;
  if (!hip_ok(hipMemcpy(out, k_out, 2 * rows * sizeof(uint16_t), hipMemcpyDeviceToHost), "hipMemcpy back")) return 1;
  f = fopen(argv[2], "wb");
  if (!f || fwrite(out, sizeof(uint16_t), 2 * rows, f) != 2 * rows) return 1;
  fclose(f);
  if (ws) (void)hipFree(ws);
  (void)hipFree(dev);
  free(host);
  free(out);
  printf("rehydrate_demo: %s, %lld tokens x %d layers rehydrated at delta %lld%s\n", kamera_version(), (long long)T,
         LAYERS, (long long)delta, noalloc ? " (no workspace)" : "");
  return 0;
}
