/*
 * A plain C caller of libringattn (C99, no C++ and no Python): the fused ring
 * forward of ra_ring_fwd through the C ABI of include/ringattn.h, with device
 * memory from the HIP runtime.  Used by tests/test_gpu_c_abi.py, which writes
 * the inputs (seeded bf16 draws in chunk-major order), runs this program and
 * compares its outputs with the float64 oracle.
 *
 * usage: ring_fwd_example DIR
 *   DIR/meta.txt   "batch hq hkv seq n_chunks layout causal"
 *   DIR/q.bin, k.bin, v.bin   bf16 [batch, heads, seq, 128], chunk-major rows
 *   writes DIR/out.bin (bf16, like q) and DIR/lse.bin (fp32 [batch, hq, seq])
 * Exit status 0 on success; a rejected call or a HIP error prints the
 * library's message and exits non-zero.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ringattn.h"

static int load(const char* dir, const char* name, void* buf, size_t bytes) {
  char path[4096];
  FILE* f;
  size_t got;
  snprintf(path, sizeof path, "%s/%s", dir, name);
  f = fopen(path, "rb");
  if (!f) return -1;
  got = fread(buf, 1, bytes, f);
  fclose(f);
  return got == bytes ? 0 : -1;
}

static int save(const char* dir, const char* name, const void* buf, size_t bytes) {
  char path[4096];
  FILE* f;
  size_t put;
  snprintf(path, sizeof path, "%s/%s", dir, name);
  f = fopen(path, "wb");
  if (!f) return -1;
  put = fwrite(buf, 1, bytes, f);
  fclose(f);
  return put == bytes ? 0 : -1;
}

#define HIP_OK(call)                                                          \
  do {                                                                        \
    hipError_t e_ = (call);                                                   \
    if (e_ != hipSuccess) {                                                   \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));       \
      return 3;                                                               \
    }                                                                         \
  } while (0)

static ra_strides contiguous(int64_t heads, int64_t rows, int64_t d) {
  ra_strides s;
  s.b = heads * rows * d;
  s.h = rows * d;
  s.s = d;
  return s;
}

int main(int argc, char** argv) {
  const int64_t d = 128;
  long long batch, hq, hkv, seq, n_chunks, layout, causal;
  char path[4096];
  FILE* meta;
  size_t q_bytes, kv_bytes, lse_bytes;
  void *hq_buf, *hk_buf, *hv_buf, *hout_buf, *hlse_buf;
  void *q, *k, *v, *out;
  float* lse;
  ra_ring_desc desc;
  ra_status st;

  if (argc != 2) {
    fprintf(stderr, "usage: %s DIR\n", argv[0]);
    return 1;
  }
  snprintf(path, sizeof path, "%s/meta.txt", argv[1]);
  meta = fopen(path, "r");
  if (!meta || fscanf(meta, "%lld %lld %lld %lld %lld %lld %lld", &batch, &hq, &hkv, &seq, &n_chunks, &layout,
                      &causal) != 7) {
    fprintf(stderr, "cannot read %s\n", path);
    return 1;
  }
  fclose(meta);
  if (ra_abi_version() != RA_ABI_VERSION) {
    fprintf(stderr, "library ABI %d, header %d\n", ra_abi_version(), RA_ABI_VERSION);
    return 1;
  }

  q_bytes = (size_t)(batch * hq * seq * d * 2);
  kv_bytes = (size_t)(batch * hkv * seq * d * 2);
  lse_bytes = (size_t)(batch * hq * seq * 4);
  hq_buf = malloc(q_bytes);
  hk_buf = malloc(kv_bytes);
  hv_buf = malloc(kv_bytes);
  hout_buf = malloc(q_bytes);
  hlse_buf = malloc(lse_bytes);
  if (!hq_buf || !hk_buf || !hv_buf || !hout_buf || !hlse_buf) return 1;
  if (load(argv[1], "q.bin", hq_buf, q_bytes) || load(argv[1], "k.bin", hk_buf, kv_bytes) ||
      load(argv[1], "v.bin", hv_buf, kv_bytes)) {
    fprintf(stderr, "cannot read the inputs\n");
    return 1;
  }

  HIP_OK(hipMalloc(&q, q_bytes));
  HIP_OK(hipMalloc(&k, kv_bytes));
  HIP_OK(hipMalloc(&v, kv_bytes));
  HIP_OK(hipMalloc(&out, q_bytes));
  HIP_OK(hipMalloc((void**)&lse, lse_bytes));
  HIP_OK(hipMemcpy(q, hq_buf, q_bytes, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(k, hk_buf, kv_bytes, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(v, hv_buf, kv_bytes, hipMemcpyHostToDevice));

  /* every query chunk, bf16 in and out, lse in natural log */
  memset(&desc, 0, sizeof desc);
  desc.attn.batch = batch;
  desc.attn.hq = hq;
  desc.attn.hkv = hkv;
  desc.attn.lq = desc.attn.lk = seq / n_chunks;
  desc.attn.d = d;
  desc.attn.in_dtype = RA_BF16;
  desc.attn.out_dtype = RA_BF16;
  desc.attn.q = contiguous(hq, seq, d);
  desc.attn.k = contiguous(hkv, seq, d);
  desc.attn.v = contiguous(hkv, seq, d);
  desc.attn.out = contiguous(hq, seq, d);
  desc.attn.ml = contiguous(hq, seq, 1);
  desc.attn.scale = 0.f;
  desc.seq = seq;
  desc.n_chunks = (int32_t)n_chunks;
  desc.layout = (int32_t)layout;
  desc.causal = (int32_t)causal;
  desc.q_chunk_first = 0;
  desc.q_chunk_count = (int32_t)n_chunks;
  desc.kv_splits = 0;

  /* a rejected call enqueues nothing and says why */
  st = ra_ring_fwd(&desc, NULL, k, v, out, lse, NULL, 0, NULL);
  if (st != RA_ERR_INVALID_ARG || strlen(ra_last_error()) == 0) {
    fprintf(stderr, "a NULL q was not rejected (%s)\n", ra_status_str(st));
    return 4;
  }
  if (ra_ring_workspace_bytes(&desc) != 0) {
    fprintf(stderr, "no workspace expected without split-KV\n");
    return 4;
  }
  st = ra_ring_fwd(&desc, q, k, v, out, lse, NULL, 0, NULL);
  if (st != RA_OK) {
    fprintf(stderr, "ra_ring_fwd: %s: %s\n", ra_status_str(st), ra_last_error());
    return 2;
  }
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(hout_buf, out, q_bytes, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hlse_buf, lse, lse_bytes, hipMemcpyDeviceToHost));
  if (save(argv[1], "out.bin", hout_buf, q_bytes) || save(argv[1], "lse.bin", hlse_buf, lse_bytes)) {
    fprintf(stderr, "cannot write the outputs\n");
    return 1;
  }
  HIP_OK(hipFree(q));
  HIP_OK(hipFree(k));
  HIP_OK(hipFree(v));
  HIP_OK(hipFree(out));
  HIP_OK(hipFree(lse));
  free(hq_buf);
  free(hk_buf);
  free(hv_buf);
  free(hout_buf);
  free(hlse_buf);
  printf("ok\n");
  return 0;
}
