/* The C ABI on the GPU from plain C: quantise-append K/V rows into a TBQ4
 * cache and run split-K decode attention, with device memory and copies from
 * the HIP runtime's C API and nothing else.
 *
 * Usage: abi_gpu_decode DIR B H HQ CAPACITY N_CTX N_SPLITS SIGN_SEED SCALE
 *   reads  DIR/k.bin, DIR/v.bin  fp32 [B][N_CTX][H][128]
 *          DIR/q.bin             fp32 [B][HQ][128]
 *   writes DIR/kc.bin, DIR/vc.bin the packed caches [B][H][CAPACITY][66]
 *          DIR/out.bin           fp32 [B][HQ][128]
 *          DIR/kc_step.bin, DIR/vc_step.bin, DIR/out_step.bin  the same from
 *          a second cache filled with tokens 0 .. N_CTX-2 and then one
 *          tbq4_decode_step call for token N_CTX-1 (append + attend)
 * Also checks that an over-long context is refused on the host
 * (TBQ4_ERR_CAPACITY).  Prints "ok" and exits 0, or names the failed step
 * and exits 1.  Run by tests/test_gpu_abi_c.py, which checks the outputs
 * against the oracle. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "tbq4.h"

static void die(const char *what, int code) {
  printf("FAILED %s (%d)\n", what, code);
  exit(1);
}

static void *read_file(const char *dir, const char *name, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE *f = fopen(path, "rb");
  if (!f) die(path, 0);
  void *p = malloc(bytes);
  if (!p || fread(p, 1, bytes, f) != bytes) die(path, 1);
  fclose(f);
  return p;
}

static void write_file(const char *dir, const char *name, const void *p, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE *f = fopen(path, "wb");
  if (!f || fwrite(p, 1, bytes, f) != bytes) die(path, 2);
  fclose(f);
}

static void *dev_alloc(size_t bytes) {
  void *p = NULL;
  hipError_t e = hipMalloc(&p, bytes);
  if (e != hipSuccess) die("hipMalloc", (int)e);
  return p;
}

int main(int argc, char **argv) {
  if (argc != 10) die("usage: DIR B H HQ CAPACITY N_CTX N_SPLITS SIGN_SEED SCALE", argc);
  const char *dir = argv[1];
  const int32_t B = atoi(argv[2]), H = atoi(argv[3]), HQ = atoi(argv[4]);
  const int32_t cap = atoi(argv[5]), n_ctx = atoi(argv[6]), n_splits = atoi(argv[7]);
  const uint64_t seed = strtoull(argv[8], NULL, 10);
  const float scale = strtof(argv[9], NULL);

  const size_t kv_bytes = (size_t)B * n_ctx * H * TBQ4_HEAD_DIM * sizeof(float);
  const size_t q_bytes = (size_t)B * HQ * TBQ4_HEAD_DIM * sizeof(float);
  const size_t cache_bytes = tbq4_cache_bytes(B, H, cap);
  const size_t ws_bytes = tbq4_decode_workspace_bytes(B, H, HQ, n_ctx, n_splits);
  if (cache_bytes == 0 || ws_bytes == 0) die("sizes", 0);

  void *k_h = read_file(dir, "k.bin", kv_bytes);
  void *v_h = read_file(dir, "v.bin", kv_bytes);
  void *q_h = read_file(dir, "q.bin", q_bytes);

  void *k_d = dev_alloc(kv_bytes), *v_d = dev_alloc(kv_bytes), *q_d = dev_alloc(q_bytes);
  void *out_d = dev_alloc(q_bytes), *ws_d = dev_alloc(ws_bytes);
  uint8_t *kc_d = (uint8_t *)dev_alloc(cache_bytes), *vc_d = (uint8_t *)dev_alloc(cache_bytes);
  if (hipMemset(kc_d, 0, cache_bytes) != hipSuccess || hipMemset(vc_d, 0, cache_bytes) != hipSuccess)
    die("hipMemset", 0);
  if (hipMemcpy(k_d, k_h, kv_bytes, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(v_d, v_h, kv_bytes, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(q_d, q_h, q_bytes, hipMemcpyHostToDevice) != hipSuccess)
    die("hipMemcpy to device", 0);

  tbq4_cache cache;
  memset(&cache, 0, sizeof cache);
  cache.k = kc_d;
  cache.v = vc_d;
  cache.batch = B;
  cache.n_kv_heads = H;
  cache.head_dim = TBQ4_HEAD_DIM;
  cache.capacity = cap;
  cache.sign_seed = seed;

  tbq4_status st = tbq4_quantize_append(&cache, k_d, v_d, TBQ4_F32, 0, n_ctx, NULL);
  if (st != TBQ4_OK) die("tbq4_quantize_append", st);
  st = tbq4_attn_decode(&cache, q_d, TBQ4_F32, HQ, n_ctx, scale, out_d, TBQ4_F32, n_splits, ws_d,
                        ws_bytes, NULL);
  if (st != TBQ4_OK) die("tbq4_attn_decode", st);
  /* refused before anything is launched */
  st = tbq4_attn_decode(&cache, q_d, TBQ4_F32, HQ, cap + 8, scale, out_d, TBQ4_F32, n_splits, ws_d,
                        ws_bytes, NULL);
  if (st != TBQ4_ERR_CAPACITY) die("over-long context not refused", st);
  if (hipDeviceSynchronize() != hipSuccess) die("hipDeviceSynchronize", 0);

  /* the decode step on a second cache: tokens 0 .. n_ctx-2 appended, then the
     last token appended and attended by one tbq4_decode_step call */
  const size_t row_bytes = (size_t)H * TBQ4_HEAD_DIM * sizeof(float);   /* one token, all heads */
  const size_t step_ws_bytes = tbq4_decode_step_workspace_bytes(B, H, HQ, n_ctx, n_splits);
  if (step_ws_bytes == 0) die("step workspace size", 0);
  uint8_t *kc2_d = (uint8_t *)dev_alloc(cache_bytes), *vc2_d = (uint8_t *)dev_alloc(cache_bytes);
  void *ws2_d = dev_alloc(step_ws_bytes), *out2_d = dev_alloc(q_bytes);
  void *kp_d = dev_alloc(kv_bytes), *vp_d = dev_alloc(kv_bytes);
  void *kl_d = dev_alloc((size_t)B * row_bytes), *vl_d = dev_alloc((size_t)B * row_bytes);
  if (hipMemset(kc2_d, 0, cache_bytes) != hipSuccess || hipMemset(vc2_d, 0, cache_bytes) != hipSuccess)
    die("hipMemset", 1);
  for (int32_t b = 0; b < B; ++b) {   /* [B][n_ctx-1][H][128] prefix and [B][1][H][128] last token */
    const char *kb = (const char *)k_h + (size_t)b * n_ctx * row_bytes;
    const char *vb = (const char *)v_h + (size_t)b * n_ctx * row_bytes;
    const size_t pre = (size_t)(n_ctx - 1) * row_bytes;
    if (hipMemcpy((char *)kp_d + (size_t)b * pre, kb, pre, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy((char *)vp_d + (size_t)b * pre, vb, pre, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy((char *)kl_d + (size_t)b * row_bytes, kb + pre, row_bytes, hipMemcpyHostToDevice) !=
            hipSuccess ||
        hipMemcpy((char *)vl_d + (size_t)b * row_bytes, vb + pre, row_bytes, hipMemcpyHostToDevice) !=
            hipSuccess)
      die("hipMemcpy step inputs", 0);
  }
  tbq4_cache cache2 = cache;
  cache2.k = kc2_d;
  cache2.v = vc2_d;
  if (n_ctx > 1) {
    st = tbq4_quantize_append(&cache2, kp_d, vp_d, TBQ4_F32, 0, n_ctx - 1, NULL);
    if (st != TBQ4_OK) die("tbq4_quantize_append (prefix)", st);
  }
  st = tbq4_decode_step(&cache2, kl_d, vl_d, TBQ4_F32, n_ctx - 1, NULL, q_d, TBQ4_F32, HQ, scale,
                        out2_d, TBQ4_F32, n_splits, ws2_d, step_ws_bytes, NULL);
  if (st != TBQ4_OK) die("tbq4_decode_step", st);
  /* the step's workspace is one partial state per head larger than the decode's */
  st = tbq4_decode_step(&cache2, kl_d, vl_d, TBQ4_F32, n_ctx - 1, NULL, q_d, TBQ4_F32, HQ, scale,
                        out2_d, TBQ4_F32, n_splits, ws2_d, step_ws_bytes - 256, NULL);
  if (st != TBQ4_ERR_WORKSPACE) die("short step workspace not refused", st);
  if (hipDeviceSynchronize() != hipSuccess) die("hipDeviceSynchronize (step)", 0);

  void *kc_h = malloc(cache_bytes), *vc_h = malloc(cache_bytes), *out_h = malloc(q_bytes);
  if (!kc_h || !vc_h || !out_h) die("malloc", 0);
  if (hipMemcpy(kc_h, kc_d, cache_bytes, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(vc_h, vc_d, cache_bytes, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(out_h, out_d, q_bytes, hipMemcpyDeviceToHost) != hipSuccess)
    die("hipMemcpy to host", 0);
  write_file(dir, "kc.bin", kc_h, cache_bytes);
  write_file(dir, "vc.bin", vc_h, cache_bytes);
  write_file(dir, "out.bin", out_h, q_bytes);
  if (hipMemcpy(kc_h, kc2_d, cache_bytes, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(vc_h, vc2_d, cache_bytes, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(out_h, out2_d, q_bytes, hipMemcpyDeviceToHost) != hipSuccess)
    die("hipMemcpy to host (step)", 0);
  write_file(dir, "kc_step.bin", kc_h, cache_bytes);
  write_file(dir, "vc_step.bin", vc_h, cache_bytes);
  write_file(dir, "out_step.bin", out_h, q_bytes);

  hipFree(k_d);
  hipFree(v_d);
  hipFree(q_d);
  hipFree(out_d);
  hipFree(ws_d);
  hipFree(kc_d);
  hipFree(vc_d);
  hipFree(kc2_d);
  hipFree(vc2_d);
  hipFree(ws2_d);
  hipFree(out2_d);
  hipFree(kp_d);
  hipFree(vp_d);
  hipFree(kl_d);
  hipFree(vl_d);
  free(k_h);
  free(v_h);
  free(q_h);
  free(kc_h);
  free(vc_h);
  free(out_h);
  printf("ok\n");
  return 0;
}
