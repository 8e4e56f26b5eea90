/*
 * A C caller of libfp8kv.so, with no Python or torch in the process: reads the
 * inputs of one fused-prologue call from a file, runs the call on a HIP
 * stream of its own, and writes q, the cache and the exponent rows back.
 *
 *   c_abi_driver IN OUT
 *
 * IN:  int64 T, H, pages, max_position; double eps; then, little-endian and
 *      densely packed: q bf16[T*H*512], kv bf16[T*512], q_weight bf16[512],
 *      kv_weight bf16[512], cos_sin fp32[max_position*64], positions
 *      int64[T], slot_mapping int64[T], kv_cache u8[pages*64*576],
 *      kv_scale u8[pages*64*8]
 * OUT: q, kv_cache, kv_scale after the call, in that order; then, when the
 *      cache has pages, the cache read back through a block table (one
 *      sequence covering every page in order): bf16[pages*64*512].
 *
 * Before the real call it makes one call with a NULL kv pointer and checks
 * that the library refuses it (FP8KV_ERR_NULL) with a status string.  Exit
 * status 0 on success; any HIP or library error prints a message and exits
 * non-zero.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fp8kv.h"

#define CHECK_HIP(x)                                                        \
  do {                                                                      \
    hipError_t e_ = (x);                                                    \
    if (e_ != hipSuccess) {                                                 \
      fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));               \
      exit(2);                                                              \
    }                                                                       \
  } while (0)

static void* read_exact(FILE* f, size_t n) {
  void* p = malloc(n ? n : 1);
  if (!p || fread(p, 1, n, f) != n) {
    fprintf(stderr, "short input\n");
    exit(3);
  }
  return p;
}

static void* to_device(const void* h, size_t n) {
  void* d = NULL;
  CHECK_HIP(hipMalloc(&d, n ? n : 16));
  if (n) CHECK_HIP(hipMemcpy(d, h, n, hipMemcpyHostToDevice));
  return d;
}

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s IN OUT\n", argv[0]);
    return 1;
  }
  FILE* in = fopen(argv[1], "rb");
  if (!in) {
    perror(argv[1]);
    return 1;
  }
  int64_t hdr[4];
  double eps;
  if (fread(hdr, sizeof hdr, 1, in) != 1 || fread(&eps, sizeof eps, 1, in) != 1) {
    fprintf(stderr, "short header\n");
    return 3;
  }
  const int64_t T = hdr[0], H = hdr[1], pages = hdr[2], maxp = hdr[3];
  const size_t nq = (size_t)(T * H * 512 * 2), nkv = (size_t)(T * 512 * 2);
  const size_t ncs = (size_t)(maxp * 64 * 4), nidx = (size_t)(T * 8);
  const size_t ncache = (size_t)(pages * 64 * 576), nscale = (size_t)(pages * 64 * 8);
  void* hq = read_exact(in, nq);
  void* hkv = read_exact(in, nkv);
  void* hqw = read_exact(in, 1024);
  void* hkw = read_exact(in, 1024);
  void* hcs = read_exact(in, ncs);
  void* hpos = read_exact(in, nidx);
  void* hslot = read_exact(in, nidx);
  void* hcache = read_exact(in, ncache);
  void* hscale = read_exact(in, nscale);
  fclose(in);

  void* q = to_device(hq, nq);
  void* kv = to_device(hkv, nkv);
  void* qw = to_device(hqw, 1024);
  void* kw = to_device(hkw, 1024);
  void* cs = to_device(hcs, ncs);
  void* pos = to_device(hpos, nidx);
  void* slot = to_device(hslot, nidx);
  void* cache = to_device(hcache, ncache);
  void* scale = to_device(hscale, nscale);
  hipStream_t stream;
  CHECK_HIP(hipStreamCreate(&stream));

  if (fp8kv_abi_version() != FP8KV_ABI_VERSION) {
    fprintf(stderr, "ABI version mismatch\n");
    return 4;
  }
  int st = qnorm_rope_kv_quant_insert(
      q, NULL, qw, kw, (const float*)cs, (const int64_t*)pos,
      (const int64_t*)slot, (uint8_t*)cache, (uint8_t*)scale, T, (int32_t)H,
      512, 64, maxp, pages, 64, (float)eps, (void*)stream);
  if (st != FP8KV_ERR_NULL || !fp8kv_status_string(st)[0]) {
    fprintf(stderr, "NULL kv not refused: status %d\n", st);
    return 5;
  }
  st = qnorm_rope_kv_quant_insert(
      q, kv, qw, kw, (const float*)cs, (const int64_t*)pos, (const int64_t*)slot,
      (uint8_t*)cache, (uint8_t*)scale, T, (int32_t)H, 512, 64, maxp, pages, 64,
      (float)eps, (void*)stream);
  if (st != FP8KV_OK) {
    fprintf(stderr, "call failed: %s\n", fp8kv_status_string(st));
    return 6;
  }
  /* read the cache back through a block table on the same stream */
  const size_t nrows = (size_t)(pages * 64), nread = nrows * 512 * 2;
  void* hread = malloc(nread ? nread : 1);
  void* dread = NULL;
  if (pages > 0) {
    int32_t* htable = (int32_t*)malloc((size_t)pages * sizeof(int32_t));
    if (!hread || !htable) {
      fprintf(stderr, "out of host memory\n");
      return 8;
    }
    for (int64_t i = 0; i < pages; ++i) htable[i] = (int32_t)i;
    const int32_t hlen = (int32_t)nrows;
    const int64_t hoff = 0;
    void* dtable = to_device(htable, (size_t)pages * sizeof(int32_t));
    void* dlen = to_device(&hlen, sizeof hlen);
    void* doff = to_device(&hoff, sizeof hoff);
    CHECK_HIP(hipMalloc(&dread, nread));
    st = kv_cache_gather_dequant_paged(
        (const uint8_t*)cache, (const uint8_t*)scale, pages, 64,
        (const int32_t*)dtable, 1, (int32_t)pages, (const int32_t*)dlen,
        (const int64_t*)doff, (int64_t)nrows, dread, (void*)stream);
    if (st != FP8KV_OK) {
      fprintf(stderr, "read-back failed: %s\n", fp8kv_status_string(st));
      return 9;
    }
    CHECK_HIP(hipStreamSynchronize(stream));
    CHECK_HIP(hipMemcpy(hread, dread, nread, hipMemcpyDeviceToHost));
    CHECK_HIP(hipFree(dtable));
    CHECK_HIP(hipFree(dlen));
    CHECK_HIP(hipFree(doff));
    CHECK_HIP(hipFree(dread));
    free(htable);
  }
  CHECK_HIP(hipStreamSynchronize(stream));
  CHECK_HIP(hipMemcpy(hq, q, nq, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(hcache, cache, ncache, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(hscale, scale, nscale, hipMemcpyDeviceToHost));

  FILE* out = fopen(argv[2], "wb");
  if (!out || fwrite(hq, 1, nq, out) != nq || fwrite(hcache, 1, ncache, out) != ncache ||
      fwrite(hscale, 1, nscale, out) != nscale ||
      (pages > 0 && fwrite(hread, 1, nread, out) != nread)) {
    fprintf(stderr, "cannot write %s\n", argv[2]);
    return 7;
  }
  fclose(out);
  free(hread);
  CHECK_HIP(hipStreamDestroy(stream));
  void* dev[] = {q, kv, qw, kw, cs, pos, slot, cache, scale};
  for (size_t i = 0; i < sizeof dev / sizeof dev[0]; ++i) CHECK_HIP(hipFree(dev[i]));
  void* host[] = {hq, hkv, hqw, hkw, hcs, hpos, hslot, hcache, hscale};
  for (size_t i = 0; i < sizeof host / sizeof host[0]; ++i) free(host[i]);
  return 0;
}
