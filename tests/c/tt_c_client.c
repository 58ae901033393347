/* A plain C99 client of libtt.so: the library's C ABI used the way a C or
 * C++ caller outside Python would use it (include/tt.h, device memory from
 * the HIP runtime, no torch).  Built by the package build with gcc.
 *
 *   tt_c_client host
 *       Calls that need no GPU: version, status strings, workspace queries and
 *       the argument checks that reject a call before any HIP call.  Prints
 *       one "name value" line per result.
 *   tt_c_client gpu DIR
 *       One denoising step on the first GPU.  Reads DIR/shape.txt
 *       ("B Hq Hkv L P D k V scale") and the inputs q.bin, k_ctx.bin,
 *       v_ctx.bin, k_blk.bin, v_blk.bin (bf16 bit patterns), logits.bin (fp32),
 *       mask.bin (uint8), tokens.bin (int32); runs tt_block_attn (bf16 output)
 *       and tt_unmask_step (fixed k, with its confidence and prediction
 *       outputs) on one stream; writes out.bin, tokens_out.bin, mask_out.bin,
 *       conf.bin and pred.bin.  Exits with status 1 on any error, after
 *       printing it.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "tt.h"

#define CHECK_HIP(call)                                                      \
  do {                                                                       \
    hipError_t e_ = (call);                                                  \
    if (e_ != hipSuccess) {                                                  \
      fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));             \
      return 1;                                                              \
    }                                                                        \
  } while (0)

#define CHECK_TT(call)                                                       \
  do {                                                                       \
    tt_status s_ = (call);                                                   \
    if (s_ != TT_OK) {                                                       \
      fprintf(stderr, "%s: %s\n", #call, tt_status_string(s_));              \
      return 1;                                                              \
    }                                                                        \
  } while (0)

static int host_mode(void) {
  /* A pointer value that is never dereferenced: every call below fails its
   * argument checks first. */
  void* fake = (void*)(uintptr_t)0x1000;
  printf("version %s\n", tt_version());
  printf("status_ok %s\n", tt_status_string(TT_OK));
  printf("status_einval %s\n", tt_status_string(TT_EINVAL));
  printf("attn_ws_decode %zu\n",
         tt_block_attn_workspace_bytes(8, 2048, 32, 32, 2, 128, TT_BF16, NULL));
  printf("attn_ws_highbatch %zu\n",
         tt_block_attn_workspace_bytes(64, 4096, 64, 32, 2, 128, TT_BF16, NULL));
  printf("attn_ws_bad_heads %d\n",
         tt_block_attn_workspace_bytes(8, 2048, 32, 3, 2, 128, TT_BF16, NULL) == SIZE_MAX);
  printf("unmask_ws_decode %zu\n", tt_unmask_workspace_bytes(8, 32, 131072));
  /* n_q_heads not a multiple of n_kv_heads */
  printf("attn_bad_heads %d\n",
         (int)tt_block_attn(fake, fake, fake, 16, fake, fake, 16, 3, 2, 128, 0.088f, fake, 1, 16,
                            TT_BF16, TT_BF16, NULL, 0, 0));
  /* prefix_len beyond the cache capacity */
  printf("attn_prefix_over_cap %d\n",
         (int)tt_block_attn(fake, fake, fake, 32, fake, fake, 16, 4, 2, 128, 0.088f, fake, 1, 16,
                            TT_BF16, TT_BF16, NULL, 0, 0));
  /* null output */
  printf("attn_null_out %d\n",
         (int)tt_block_attn(fake, fake, fake, 16, fake, fake, 16, 4, 2, 128, 0.088f, NULL, 1, 16,
                            TT_BF16, TT_BF16, NULL, 0, 0));
  /* negative k */
  printf("unmask_negative_k %d\n",
         (int)tt_unmask_step((const float*)fake, (const uint8_t*)fake, -1, (int32_t*)fake,
                             (uint8_t*)fake, 2, 16, 1000, NULL, NULL, fake, 1 << 20, 0));
  /* workspace too small */
  printf("unmask_short_workspace %d\n",
         (int)tt_unmask_step((const float*)fake, (const uint8_t*)fake, 4, (int32_t*)fake,
                             (uint8_t*)fake, 2, 16, 1000, NULL, NULL, fake, 1, 0));
  return 0;
}

static void* read_file(const char* dir, const char* name, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) {
    fprintf(stderr, "cannot open %s\n", path);
    return NULL;
  }
  void* buf = malloc(bytes ? bytes : 1);
  size_t got = bytes ? fread(buf, 1, bytes, f) : 0;
  fclose(f);
  if (got != bytes) {
    fprintf(stderr, "%s: read %zu of %zu bytes\n", path, got, bytes);
    free(buf);
    return NULL;
  }
  return buf;
}

static int write_file(const char* dir, const char* name, const void* buf, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "wb");
  if (!f) return 1;
  size_t put = fwrite(buf, 1, bytes, f);
  fclose(f);
  return put != bytes;
}

/* Host buffer -> new device buffer of the same size. */
static int upload(const char* dir, const char* name, size_t bytes, void** dev) {
  void* h = read_file(dir, name, bytes);
  if (!h) return 1;
  CHECK_HIP(hipMalloc(dev, bytes ? bytes : 16));
  CHECK_HIP(hipMemcpy(*dev, h, bytes, hipMemcpyHostToDevice));
  free(h);
  return 0;
}

static int gpu_mode(const char* dir) {
  int B, Hq, Hkv, L, P, D, k, V;
  float scale;
  {
    char path[4096];
    snprintf(path, sizeof path, "%s/shape.txt", dir);
    FILE* f = fopen(path, "r");
    if (!f || fscanf(f, "%d %d %d %d %d %d %d %d %f", &B, &Hq, &Hkv, &L, &P, &D, &k, &V,
                     &scale) != 9) {
      fprintf(stderr, "bad %s\n", path);
      return 1;
    }
    fclose(f);
  }
  const size_t q_bytes = (size_t)B * Hq * L * D * 2;
  const size_t ctx_bytes = (size_t)B * Hkv * P * D * 2;
  const size_t blk_bytes = (size_t)B * Hkv * L * D * 2;
  const size_t lg_bytes = (size_t)B * L * V * 4;
  const size_t pos = (size_t)B * L;
  void *q, *kc, *vc, *kb, *vb, *lg, *mask, *tok, *out, *mask_out, *conf, *pred, *ws_a = NULL, *ws_u;
  if (upload(dir, "q.bin", q_bytes, &q) || upload(dir, "k_ctx.bin", ctx_bytes, &kc) ||
      upload(dir, "v_ctx.bin", ctx_bytes, &vc) || upload(dir, "k_blk.bin", blk_bytes, &kb) ||
      upload(dir, "v_blk.bin", blk_bytes, &vb) || upload(dir, "logits.bin", lg_bytes, &lg) ||
      upload(dir, "mask.bin", pos, &mask) || upload(dir, "tokens.bin", pos * 4, &tok))
    return 1;
  CHECK_HIP(hipMalloc(&out, q_bytes));
  CHECK_HIP(hipMalloc(&mask_out, pos));
  CHECK_HIP(hipMalloc(&conf, pos * 4));
  CHECK_HIP(hipMalloc(&pred, pos * 4));
  const size_t ws_a_bytes = tt_block_attn_workspace_bytes(B, P, L, Hq, Hkv, D, TT_BF16, NULL);
  const size_t ws_u_bytes = tt_unmask_workspace_bytes(B, L, V);
  if (ws_a_bytes == SIZE_MAX || ws_u_bytes == SIZE_MAX) {
    fprintf(stderr, "invalid shape\n");
    return 1;
  }
  if (ws_a_bytes) CHECK_HIP(hipMalloc(&ws_a, ws_a_bytes));
  CHECK_HIP(hipMalloc(&ws_u, ws_u_bytes));
  hipStream_t stream;
  CHECK_HIP(hipStreamCreate(&stream));

  CHECK_TT(tt_block_attn(q, P ? kc : NULL, P ? vc : NULL, P, kb, vb, L, Hq, Hkv, D, scale, out,
                         B, P, TT_BF16, TT_BF16, ws_a, ws_a_bytes, stream));
  CHECK_TT(tt_unmask_step((const float*)lg, (const uint8_t*)mask, k, (int32_t*)tok,
                          (uint8_t*)mask_out, B, L, V, (float*)conf, (int32_t*)pred, ws_u,
                          ws_u_bytes, stream));
  CHECK_HIP(hipStreamSynchronize(stream));

  void* h_out = malloc(q_bytes);
  void* h_tok = malloc(pos * 4);
  void* h_mask = malloc(pos);
  void* h_conf = malloc(pos * 4);
  void* h_pred = malloc(pos * 4);
  CHECK_HIP(hipMemcpy(h_out, out, q_bytes, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(h_tok, tok, pos * 4, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(h_mask, mask_out, pos, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(h_conf, conf, pos * 4, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(h_pred, pred, pos * 4, hipMemcpyDeviceToHost));
  if (write_file(dir, "out.bin", h_out, q_bytes) ||
      write_file(dir, "tokens_out.bin", h_tok, pos * 4) ||
      write_file(dir, "mask_out.bin", h_mask, pos) || write_file(dir, "conf.bin", h_conf, pos * 4) ||
      write_file(dir, "pred.bin", h_pred, pos * 4)) {
    fprintf(stderr, "cannot write outputs to %s\n", dir);
    return 1;
  }
  free(h_out);
  free(h_tok);
  free(h_mask);
  free(h_conf);
  free(h_pred);
  void* bufs[] = {q, kc, vc, kb, vb, lg, mask, tok, out, mask_out, conf, pred, ws_u};
  for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i) CHECK_HIP(hipFree(bufs[i]));
  if (ws_a) CHECK_HIP(hipFree(ws_a));
  CHECK_HIP(hipStreamDestroy(stream));
  printf("gpu step ok\n");
  return 0;
}

int main(int argc, char** argv) {
  if (argc == 2 && strcmp(argv[1], "host") == 0) return host_mode();
  if (argc == 3 && strcmp(argv[1], "gpu") == 0) return gpu_mode(argv[2]);
  fprintf(stderr, "usage: %s host | %s gpu DIR\n", argv[0], argv[0]);
  return 2;
}
