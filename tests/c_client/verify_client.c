/*
 * A plain C client of libspec_verify.so (no Python, no PyTorch): reads one
 * packed batch from a file, runs spec_verify_run on device buffers it
 * allocates with the HIP runtime, and writes the outputs to a file.  The GPU
 * tests run it as a child process and compare its outputs with the oracle.
 *
 * Input (little-endian): "SVC1", int32 B, int64 R_d, int64 V, int32 dtype
 * (0 f32, 1 bf16), float T, then cu_draft[B+1] int32, target logits
 * [R_t][V], draft logits [R_d][V] (dtype), draft tokens [R_d] int32,
 * uniforms [R_t] float32, with R_t = R_d + B.
 * Output: "SVO1", out_tokens[R_t] int32, num_accepted[B] int32,
 * p_draft[R_d] float32, q_draft[R_d] float32, residual_sum[B] float32,
 * status uint32.
 * Exit status 0 on success; on any failure a message on stderr and 1.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "spec_verify.h"

static int fail(const char *what) {
  fprintf(stderr, "verify_client: %s\n", what);
  return 1;
}

static int read_all(FILE *f, void *dst, size_t n) { return fread(dst, 1, n, f) == n; }

static void *dev_copy(const void *src, size_t n) {
  void *d = NULL;
  if (hipMalloc(&d, n ? n : 4) != hipSuccess) return NULL;
  if (n && hipMemcpy(d, src, n, hipMemcpyHostToDevice) != hipSuccess) return NULL;
  return d;
}

int main(int argc, char **argv) {
  if (argc != 3) return fail("usage: verify_client <input> <output>");
  FILE *in = fopen(argv[1], "rb");
  if (!in) return fail("cannot open the input");
  char magic[4];
  int32_t B, dtype;
  int64_t R_d, V;
  float T;
  if (!read_all(in, magic, 4) || memcmp(magic, "SVC1", 4) != 0) return fail("bad input magic");
  if (!read_all(in, &B, 4) || !read_all(in, &R_d, 8) || !read_all(in, &V, 8) ||
      !read_all(in, &dtype, 4) || !read_all(in, &T, 4))
    return fail("short header");
  if (B < 1 || R_d < 0 || V < 1 || (dtype != SPEC_VERIFY_F32 && dtype != SPEC_VERIFY_BF16))
    return fail("bad header values");
  const int64_t R_t = R_d + B;
  const size_t esize = dtype == SPEC_VERIFY_BF16 ? 2 : 4;
  const size_t n_cu = (size_t)(B + 1) * 4, n_t = (size_t)R_t * (size_t)V * esize;
  const size_t n_d = (size_t)R_d * (size_t)V * esize, n_tok = (size_t)R_d * 4;
  const size_t n_u = (size_t)R_t * 4;
  void *h_cu = malloc(n_cu), *h_t = malloc(n_t), *h_d = malloc(n_d ? n_d : 1);
  void *h_tok = malloc(n_tok ? n_tok : 1), *h_u = malloc(n_u);
  if (!h_cu || !h_t || !h_d || !h_tok || !h_u) return fail("out of host memory");
  if (!read_all(in, h_cu, n_cu) || !read_all(in, h_t, n_t) || !read_all(in, h_d, n_d) ||
      !read_all(in, h_tok, n_tok) || !read_all(in, h_u, n_u))
    return fail("short input arrays");
  fclose(in);

  if (hipSetDevice(0) != hipSuccess) return fail("hipSetDevice");
  spec_verify_ctx *ctx = NULL;
  size_t ws_bytes = 0;
  int st = spec_verify_create(&ctx, 0, V, dtype, B, R_d, 0, &ws_bytes);
  if (st != SPEC_VERIFY_OK) {
    fprintf(stderr, "verify_client: spec_verify_create: %s\n", spec_verify_status_string(st));
    return 1;
  }
  spec_verify_args a;
  memset(&a, 0, sizeof(a));
  a.num_seqs = B;
  a.total_draft_rows = R_d;
  a.cu_draft = (const int32_t *)dev_copy(h_cu, n_cu);
  a.target_logits = dev_copy(h_t, n_t);
  a.draft_logits = R_d > 0 ? dev_copy(h_d, n_d) : NULL;
  a.ld = V;
  a.draft_tokens = R_d > 0 ? (const int32_t *)dev_copy(h_tok, n_tok) : NULL;
  a.uniforms = (const float *)dev_copy(h_u, n_u);
  a.temperature = T;
  void *out_tok = NULL, *out_n = NULL, *out_p = NULL, *out_q = NULL, *out_r = NULL;
  void *status = NULL, *ws = NULL;
  if (hipMalloc(&out_tok, (size_t)R_t * 4) != hipSuccess ||
      hipMalloc(&out_n, (size_t)B * 4) != hipSuccess ||
      hipMalloc(&out_p, (size_t)(R_d ? R_d : 1) * 4) != hipSuccess ||
      hipMalloc(&out_q, (size_t)(R_d ? R_d : 1) * 4) != hipSuccess ||
      hipMalloc(&out_r, (size_t)B * 4) != hipSuccess || hipMalloc(&status, 4) != hipSuccess ||
      hipMalloc(&ws, ws_bytes) != hipSuccess)
    return fail("hipMalloc");
  if (!a.cu_draft || !a.target_logits || (R_d > 0 && (!a.draft_logits || !a.draft_tokens)) ||
      !a.uniforms)
    return fail("device copies of the inputs");
  if (hipMemset(status, 0, 4) != hipSuccess) return fail("hipMemset");
  a.out_tokens = (int32_t *)out_tok;
  a.out_num_accepted = (int32_t *)out_n;
  a.out_p_draft = (float *)out_p;
  a.out_q_draft = (float *)out_q;
  a.out_residual_sum = (float *)out_r;
  a.workspace = ws;
  a.workspace_bytes = ws_bytes;
  a.status = (uint32_t *)status;
  st = spec_verify_run(ctx, &a, NULL);
  if (st != SPEC_VERIFY_OK) {
    fprintf(stderr, "verify_client: spec_verify_run: %s (hip %d)\n",
            spec_verify_status_string(st), spec_verify_last_hip_error());
    return 1;
  }
  if (hipDeviceSynchronize() != hipSuccess) return fail("hipDeviceSynchronize");

  FILE *out = fopen(argv[2], "wb");
  if (!out) return fail("cannot open the output");
  const struct { void *d; size_t n; } parts[] = {
      {out_tok, (size_t)R_t * 4}, {out_n, (size_t)B * 4}, {out_p, (size_t)R_d * 4},
      {out_q, (size_t)R_d * 4},   {out_r, (size_t)B * 4}, {status, 4}};
  fwrite("SVO1", 1, 4, out);
  for (size_t i = 0; i < sizeof(parts) / sizeof(parts[0]); ++i) {
    void *h = malloc(parts[i].n ? parts[i].n : 1);
    if (!h || (parts[i].n && hipMemcpy(h, parts[i].d, parts[i].n, hipMemcpyDeviceToHost) != hipSuccess))
      return fail("copying the outputs back");
    if (fwrite(h, 1, parts[i].n, out) != parts[i].n) return fail("writing the output");
    free(h);
  }
  fclose(out);
  spec_verify_destroy(ctx);
  return 0;
}
