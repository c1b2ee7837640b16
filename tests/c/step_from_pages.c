/* An attention step driven from plain C through include/isd.h alone, starting from the
 * paged cache in its logical layout [num_pages][Hkv][16][D] (one row of D values per
 * token slot): the caller packs the pages with isd_pack_kv_pages, runs
 * isd_attention_step, and reads the cache back with isd_unpack_kv_pages.  No Python
 * helper touches the layout.  bf16 throughout (uint16 storage).
 *
 *   step_from_pages <in.bin> <out.bin>
 * in.bin : int32 B, N, Hq, Hkv, D, num_pages, max_pages, max_ctx_len; then q [B,R,Hq,D],
 *          k_new, v_new [B,R,Hkv,D], k_pages, v_pages [num_pages,Hkv,16,D] (uint16),
 *          page_table [B,max_pages], ctx_lens [B] (int32)
 * out.bin: out [B,R,Hq,D], then k_pages, v_pages after the step (uint16)
 * Exit status 0 on success. */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

#include "isd.h"

#define HIP_OK(x)                                                        \
  do {                                                                   \
    hipError_t e_ = (x);                                                 \
    if (e_ != hipSuccess) {                                              \
      fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));            \
      return 1;                                                          \
    }                                                                    \
  } while (0)
#define ISD_OK_(x)                                                       \
  do {                                                                   \
    isd_status s_ = (x);                                                 \
    if (s_ != ISD_OK) {                                                  \
      fprintf(stderr, "%s: %s (%s)\n", #x, isd_status_string(s_), isd_last_error()); \
      return 1;                                                          \
    }                                                                    \
  } while (0)

static void* read_n(FILE* f, size_t bytes) {
  void* p = malloc(bytes ? bytes : 1);
  if (p && fread(p, 1, bytes, f) != bytes) {
    free(p);
    return NULL;
  }
  return p;
}

static int to_device(const void* host, size_t bytes, void** dev) {
  if (hipMalloc(dev, bytes) != hipSuccess) return 1;
  return hipMemcpy(*dev, host, bytes, hipMemcpyHostToDevice) != hipSuccess;
}

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s in.bin out.bin\n", argv[0]);
    return 2;
  }
  FILE* f = fopen(argv[1], "rb");
  if (!f) return 2;
  int hdr[8];
  if (fread(hdr, sizeof(int), 8, f) != 8) return 2;
  const int B = hdr[0], N = hdr[1], Hq = hdr[2], Hkv = hdr[3], D = hdr[4], P = hdr[5], maxp = hdr[6], maxctx = hdr[7];
  const int R = 2 * N - 1;
  const size_t nq = (size_t)B * R * Hq * D, nkv = (size_t)B * R * Hkv * D, npg = (size_t)P * Hkv * 16 * D;
  uint16_t* q = read_n(f, nq * 2);
  uint16_t* kn = read_n(f, nkv * 2);
  uint16_t* vn = read_n(f, nkv * 2);
  uint16_t* kp = read_n(f, npg * 2);
  uint16_t* vp = read_n(f, npg * 2);
  int32_t* pt = read_n(f, (size_t)B * maxp * 4);
  int32_t* cl = read_n(f, (size_t)B * 4);
  fclose(f);
  if (!q || !kn || !vn || !kp || !vp || !pt || !cl) return 2;

  void *dq, *dkn, *dvn, *dkp, *dvp, *dpt, *dcl, *dkc, *dvc, *dout, *dws;
  if (to_device(q, nq * 2, &dq) || to_device(kn, nkv * 2, &dkn) || to_device(vn, nkv * 2, &dvn) ||
      to_device(kp, npg * 2, &dkp) || to_device(vp, npg * 2, &dvp) || to_device(pt, (size_t)B * maxp * 4, &dpt) ||
      to_device(cl, (size_t)B * 4, &dcl))
    return 1;
  HIP_OK(hipMalloc(&dkc, npg * 2));
  HIP_OK(hipMalloc(&dvc, npg * 2));
  HIP_OK(hipMalloc(&dout, nq * 2));
  const size_t wsb = isd_attention_workspace_bytes(B, N, Hq, Hkv, D, maxctx);
  if (wsb == 0) return 1;
  HIP_OK(hipMalloc(&dws, wsb));

  ISD_OK_(isd_pack_kv_pages(ISD_BF16, dkp, dvp, dkc, dvc, P, Hkv, D, NULL));
  ISD_OK_(isd_attention_step(ISD_BF16, dq, dkn, dvn, dkc, dvc, dpt, dcl, dout, B, N, Hq, Hkv, D, ISD_PAGE_SIZE, maxp,
                             P, maxctx, 1.0f / sqrtf((float)D), dws, wsb, NULL));
  ISD_OK_(isd_unpack_kv_pages(ISD_BF16, dkc, dvc, dkp, dvp, P, Hkv, D, NULL));
  HIP_OK(hipDeviceSynchronize());

  uint16_t* out = malloc(nq * 2);
  if (!out) return 1;
  HIP_OK(hipMemcpy(out, dout, nq * 2, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(kp, dkp, npg * 2, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(vp, dvp, npg * 2, hipMemcpyDeviceToHost));
  FILE* g = fopen(argv[2], "wb");
  if (!g) return 2;
  fwrite(out, 2, nq, g);
  fwrite(kp, 2, npg, g);
  fwrite(vp, 2, npg, g);
  fclose(g);
  printf("step from pages ok\n");
  return 0;
}
