/*
 * A plain C caller of the C ABI (include/hcr.h): reads one weight set and one batch of inputs from
 * raw little-endian files, runs hcr_read on the device, and writes out and mean back to files.
 * It uses only the HIP runtime's C API for device memory and the library's entry points.
 *
 *   hcr_read_file DIR T [pending] [inj] [q8]
 *
 * DIR holds w_down.bin (BF16 [320][10240]), w_up.bin (BF16 [10240][320]), w_norm.bin (f32 [4][2560]),
 * x.bin (f32 [T][4][2560]) and, when named on the command line, pending.bin (f32 [T][4][2560]) and
 * inj.bin (f32 [T][320]).  With q8 the weights are first turned into Q8_0 copies by hcr_quantize_q8_0
 * and the read runs on those.  The program writes DIR/out.bin (f32 [T][4][2560]) and DIR/mean.bin
 * (f32 [T][2560]) and exits 0, or prints the failing call and exits 1.
 */
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "hcr.h"

#define S HCR_STREAMS
#define D HCR_STREAM_D
#define R HCR_RANK

static int fail(const char* what, const char* detail) {
  fprintf(stderr, "hcr_read_file: %s: %s\n", what, detail);
  return 1;
}

static void* load(const char* dir, const char* name, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) return NULL;
  void* host = malloc(bytes);
  size_t got = host ? fread(host, 1, bytes, f) : 0;
  fclose(f);
  if (got != bytes) {
    free(host);
    return NULL;
  }
  void* dev = NULL;
  if (hipMalloc(&dev, bytes) != hipSuccess || hipMemcpy(dev, host, bytes, hipMemcpyHostToDevice) != hipSuccess) {
    free(host);
    return NULL;
  }
  free(host);
  return dev;
}

static int save(const char* dir, const char* name, const void* dev, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  void* host = malloc(bytes);
  if (!host || hipMemcpy(host, dev, bytes, hipMemcpyDeviceToHost) != hipSuccess) {
    free(host);
    return 1;
  }
  FILE* f = fopen(path, "wb");
  size_t put = f ? fwrite(host, 1, bytes, f) : 0;
  if (f) fclose(f);
  free(host);
  return put == bytes ? 0 : 1;
}

int main(int argc, char** argv) {
  if (argc < 3) return fail("usage", "hcr_read_file DIR T [pending] [inj] [q8]");
  const char* dir = argv[1];
  const int T = atoi(argv[2]);
  int with_pending = 0, with_inj = 0, q8 = 0;
  for (int i = 3; i < argc; ++i) {
    if (!strcmp(argv[i], "pending")) with_pending = 1;
    else if (!strcmp(argv[i], "inj")) with_inj = 1;
    else if (!strcmp(argv[i], "q8")) q8 = 1;
    else return fail("unknown option", argv[i]);
  }
  int t_max = 0;
  hcr_geometry(NULL, NULL, NULL, &t_max);
  if (T < 1 || T > t_max) return fail("T", "outside 1..t_max");

  const size_t wbytes = (size_t)R * S * D * 2, sbytes = (size_t)T * S * D * 4;
  void* w_down = load(dir, "w_down.bin", wbytes);
  void* w_up = load(dir, "w_up.bin", wbytes);
  float* w_norm = (float*)load(dir, "w_norm.bin", (size_t)S * D * 4);
  float* x = (float*)load(dir, "x.bin", sbytes);
  float* pending = with_pending ? (float*)load(dir, "pending.bin", sbytes) : NULL;
  float* inj = with_inj ? (float*)load(dir, "inj.bin", (size_t)T * R * 4) : NULL;
  if (!w_down || !w_up || !w_norm || !x || (with_pending && !pending) || (with_inj && !inj))
    return fail("inputs", "a file is missing, short, or could not be copied to the device");

  float *out = NULL, *mean = NULL;
  void* scratch = NULL;
  if (hipMalloc((void**)&out, sbytes) != hipSuccess || hipMalloc((void**)&mean, (size_t)T * D * 4) != hipSuccess ||
      hipMalloc(&scratch, hcr_scratch_bytes()) != hipSuccess)
    return fail("hipMalloc", "out, mean or scratch");

  hcr_t h = NULL;
  int rc;
  if (q8) {
    void *dc = NULL, *ds = NULL, *uc = NULL, *us = NULL;
    const size_t codes = (size_t)R * S * D, scales = codes / 32 * 2;
    if (hipMalloc(&dc, codes) != hipSuccess || hipMalloc(&ds, scales) != hipSuccess ||
        hipMalloc(&uc, codes) != hipSuccess || hipMalloc(&us, scales) != hipSuccess)
      return fail("hipMalloc", "Q8_0 copies");
    if ((rc = hcr_quantize_q8_0(w_down, R, S * D, dc, ds, NULL)) != HCR_OK ||
        (rc = hcr_quantize_q8_0(w_up, S * D, R, uc, us, NULL)) != HCR_OK)
      return fail("hcr_quantize_q8_0", hcr_strerror(rc));
    rc = hcr_create_q8_0(dc, ds, uc, us, w_norm, scratch, hcr_scratch_bytes(), &h);
  } else {
    rc = hcr_create(w_down, w_up, w_norm, scratch, hcr_scratch_bytes(), &h);
  }
  if (rc != HCR_OK) return fail("hcr_create", hcr_strerror(rc));
  if ((rc = hcr_read(h, T, x, pending, inj, out, mean, NULL)) != HCR_OK) return fail("hcr_read", hcr_strerror(rc));
  if (hipDeviceSynchronize() != hipSuccess) return fail("hipDeviceSynchronize", "the read failed on the device");
  if (save(dir, "out.bin", out, sbytes) || save(dir, "mean.bin", mean, (size_t)T * D * 4))
    return fail("outputs", "could not write out.bin or mean.bin");
  hcr_destroy(h);
  return 0;
}
