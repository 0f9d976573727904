/* One layer forward through the C ABI from a plain C program using the HIP runtime's C API:
 *   forward_c T DIR
 * reads DIR/{x,wr,wg,wu,wd}.bin (bf16 x [T,2048], fp32 W_router [64,2048], bf16 W_gate / W_up
 * [64,1024,2048], bf16 W_down [64,2048,1024]), calls olmoe_moe_forward on device buffers, and
 * writes DIR/{out,ids,probs,counts,losses}.bin.  Exit status 0 on success. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "olmoe_moe.h"

static void* read_file(const char* dir, const char* name, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) return NULL;
  void* buf = malloc(bytes ? bytes : 1);
  const size_t got = buf ? fread(buf, 1, bytes, f) : 0;
  fclose(f);
  if (got != bytes) {
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
  const size_t put = fwrite(buf, 1, bytes, f);
  fclose(f);
  return put != bytes;
}

#define HIP(call)                                                              \
  do {                                                                         \
    hipError_t e_ = (call);                                                    \
    if (e_ != hipSuccess) {                                                    \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));        \
      return 1;                                                                \
    }                                                                          \
  } while (0)

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s T DIR\n", argv[0]);
    return 2;
  }
  const int64_t T = atoll(argv[1]);
  const char* dir = argv[2];
  if (T < 1 || T > 65536) return 2;
  const size_t xb = (size_t)T * OLMOE_D * 2, wrb = (size_t)OLMOE_E * OLMOE_D * 4,
               web = (size_t)OLMOE_E * OLMOE_F * OLMOE_D * 2, rb = (size_t)T * OLMOE_K * 4;
  const char* names[5] = {"x.bin", "wr.bin", "wg.bin", "wu.bin", "wd.bin"};
  const size_t sizes[5] = {xb, wrb, web, web, web};
  void* dev[5];
  for (int i = 0; i < 5; ++i) {
    void* h = read_file(dir, names[i], sizes[i]);
    if (!h) {
      fprintf(stderr, "cannot read %s\n", names[i]);
      return 1;
    }
    HIP(hipMalloc(&dev[i], sizes[i]));
    HIP(hipMemcpy(dev[i], h, sizes[i], hipMemcpyHostToDevice));
    free(h);
  }
  void *out, *ids, *probs, *counts, *losses, *ws;
  const size_t wsb = olmoe_moe_workspace_bytes(T);
  HIP(hipMalloc(&out, xb));
  HIP(hipMalloc(&ids, rb));
  HIP(hipMalloc(&probs, rb));
  HIP(hipMalloc(&counts, OLMOE_E * 4));
  HIP(hipMalloc(&losses, 256));
  HIP(hipMalloc(&ws, wsb));
  const olmoe_status_t st = olmoe_moe_forward(dev[0], (const float*)dev[1], dev[2], dev[3], dev[4], T, out,
                                              (int32_t*)ids, (float*)probs, (int32_t*)counts, (float*)losses,
                                              (float*)losses + 1, ws, wsb, NULL);
  if (st != OLMOE_OK) {
    fprintf(stderr, "olmoe_moe_forward: status %d: %s\n", (int)st, olmoe_last_error());
    return 1;
  }
  HIP(hipDeviceSynchronize());
  const char* onames[5] = {"out.bin", "ids.bin", "probs.bin", "counts.bin", "losses.bin"};
  void* osrc[5] = {out, ids, probs, counts, losses};
  const size_t osz[5] = {xb, rb, rb, OLMOE_E * 4, 8};
  for (int i = 0; i < 5; ++i) {
    void* h = malloc(osz[i]);
    if (!h) return 1;
    HIP(hipMemcpy(h, osrc[i], osz[i], hipMemcpyDeviceToHost));
    if (write_file(dir, onames[i], h, osz[i])) return 1;
    free(h);
  }
  printf("forward through the C ABI: T=%lld ok\n", (long long)T);
  return 0;
}
