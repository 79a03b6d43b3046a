/* One compressor call made from C: no Python, no torch.  The program reads a
 * case written by tests/test_gpu_c_caller.py (case.txt with the shape and
 * sizes, raw little-endian arrays beside it), allocates device memory with
 * the HIP runtime, packs the weights, sizes and allocates the workspace,
 * runs compressor_prefill or compressor_decode on the default stream, reads
 * the device error word and writes the output rows and both state pools
 * back (out.bin, kv_out.bin, score_out.bin).  Usage: abi_c_gpu DIR.
 * Exit status 0 on success; otherwise it prints which step failed. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "compressor.h"

static const char* dir;

static void* read_file(const char* name, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) return NULL;
  void* p = malloc(bytes ? bytes : 1);
  const size_t got = bytes ? fread(p, 1, bytes, f) : 0;
  fclose(f);
  if (got != bytes) {
    free(p);
    return NULL;
  }
  return p;
}

static int write_file(const char* name, const void* p, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "wb");
  if (!f) return 0;
  const size_t put = fwrite(p, 1, bytes, f);
  fclose(f);
  return put == bytes;
}

/* device copy of file `name` (bytes long); NULL device pointer if absent
 * and not required */
static int upload(const char* name, size_t bytes, int required, void** dev) {
  *dev = NULL;
  void* host = read_file(name, bytes);
  if (!host) {
    if (required) printf("missing input %s\n", name);
    return !required;
  }
  if (hipMalloc(dev, bytes ? bytes : 1) != hipSuccess ||
      hipMemcpy(*dev, host, bytes, hipMemcpyHostToDevice) != hipSuccess) {
    printf("device copy of %s failed\n", name);
    free(host);
    return 0;
  }
  free(host);
  return 1;
}

#define STEP(cond, what)              \
  do {                                \
    if (!(cond)) {                    \
      printf("failed: %s\n", what);   \
      return 1;                       \
    }                                 \
  } while (0)

int main(int argc, char** argv) {
  STEP(argc == 2, "usage: abi_c_gpu DIR");
  dir = argv[1];
  char path[4096];
  snprintf(path, sizeof path, "%s/case.txt", dir);
  FILE* f = fopen(path, "r");
  STEP(f != NULL, "open case.txt");
  int decode, ratio, D, H, rotate, bs, nblocks, stride, T, B, out_rows, has_cu, has_kvtab;
  const int n = fscanf(f, "%d %d %d %d %d %d %d %d %d %d %d %d %d", &decode, &ratio, &D, &H,
                       &rotate, &bs, &nblocks, &stride, &T, &B, &out_rows, &has_cu, &has_kvtab);
  fclose(f);
  STEP(n == 13, "parse case.txt");
  const int coff = ratio == 4 ? 2 : 1;
  const size_t cD = (size_t)coff * D;

  compressor_shape sh;
  sh.ratio = ratio;
  sh.head_dim = D;
  sh.hidden = H;
  sh.rope_head_dim = 64;
  sh.rotate = rotate;
  sh.block_size = bs;
  sh.num_blocks = nblocks;
  sh.table_stride = stride;

  void *x, *wkv, *wgate, *ape, *gamma, *cosv, *sinv, *had, *sp, *cu, *su, *st_tab, *kv_tab, *kv,
      *sc;
  STEP(upload("x.bin", (size_t)T * H * 2, 1, &x), "x");
  STEP(upload("wkv.bin", cD * H * 2, 1, &wkv), "wkv");
  STEP(upload("wgate.bin", cD * H * 2, 1, &wgate), "wgate");
  STEP(upload("ape.bin", (size_t)ratio * cD * 4, 1, &ape), "ape");
  STEP(upload("weight.bin", (size_t)D * 2, 1, &gamma), "weight");
  STEP(upload("cos.bin", (size_t)out_rows * 64 * 2, 1, &cosv), "cos");
  STEP(upload("sin.bin", (size_t)out_rows * 64 * 2, 1, &sinv), "sin");
  STEP(upload("hadamard.bin", (size_t)D * D * 2, rotate, &had), "hadamard");
  STEP(upload("start_pos.bin", (size_t)B * 4, 0, &sp), "start_pos");
  STEP(upload("cu_seqlens.bin", (size_t)(B + 1) * 4, has_cu, &cu), "cu_seqlens");
  STEP(upload("seqused.bin", (size_t)B * 4, 0, &su), "seqused");
  STEP(upload("state_block_table.bin", (size_t)B * stride * 4, 1, &st_tab), "state table");
  STEP(upload("kv_block_table.bin", (size_t)B * stride * 4, has_kvtab, &kv_tab), "kv table");
  const size_t pool = (size_t)nblocks * bs * cD * 4;
  STEP(upload("kv_state.bin", pool, 1, &kv), "kv_state");
  STEP(upload("score_state.bin", pool, 1, &sc), "score_state");

  void *w_packed, *out, *ws;
  STEP(hipMalloc(&w_packed, 2 * cD * H * 2) == hipSuccess, "panel allocation");
  STEP(hipMalloc(&out, (size_t)out_rows * D * 2 + 2) == hipSuccess, "output allocation");
  STEP(compressor_pack_weights(&sh, wkv, wgate, w_packed, NULL) == CMP_OK, "pack weights");
  size_t wsb = 0;
  if (decode)
    STEP(compressor_decode_workspace_size(&sh, B, out_rows, &wsb) == CMP_OK, "workspace size");
  else
    STEP(compressor_prefill_workspace_size(&sh, T, B, out_rows, &wsb) == CMP_OK,
         "workspace size");
  STEP(hipMalloc(&ws, wsb) == hipSuccess, "workspace allocation");

  compressor_args a;
  memset(&a, 0, sizeof a);
  a.x = x;
  a.T = T;
  a.batch = B;
  a.cu_seqlens = (const int32_t*)cu;
  a.seqused = (const int32_t*)su;
  a.start_pos = (const int32_t*)sp;
  a.kv_state = (float*)kv;
  a.score_state = (float*)sc;
  a.kv_block_table = (const int32_t*)kv_tab;
  a.state_block_table = (const int32_t*)st_tab;
  a.w_packed = w_packed;
  a.ape = (const float*)ape;
  a.norm_weight = gamma;
  a.hadamard = had;
  a.sin = sinv;
  a.cos = cosv;
  a.out = out;
  a.out_rows = out_rows;
  a.workspace = ws;
  a.workspace_bytes = wsb;
  const int status = decode ? compressor_decode(&sh, &a, NULL) : compressor_prefill(&sh, &a, NULL);
  if (status != CMP_OK) {
    printf("call returned %s\n", compressor_status_str(status));
    return 1;
  }
  int32_t code = -1;
  STEP(compressor_last_device_error(ws, NULL, &code) == CMP_OK, "device error word");
  printf("device error word %d\n", (int)code);

  const size_t ob = (size_t)out_rows * D * 2;
  void* host = malloc(pool > ob ? pool : ob);
  STEP(hipMemcpy(host, out, ob, hipMemcpyDeviceToHost) == hipSuccess, "read output");
  STEP(write_file("out.bin", host, ob), "write out.bin");
  STEP(hipMemcpy(host, kv, pool, hipMemcpyDeviceToHost) == hipSuccess, "read kv_state");
  STEP(write_file("kv_out.bin", host, pool), "write kv_out.bin");
  STEP(hipMemcpy(host, sc, pool, hipMemcpyDeviceToHost) == hipSuccess, "read score_state");
  STEP(write_file("score_out.bin", host, pool), "write score_out.bin");
  free(host);
  printf("abi_c_gpu: ok\n");
  return code == 0 ? 0 : 2;
}
