/*
 * A plain C caller of libskiparse, built by tests/test_abi_c.py.
 *
 *   c_caller plan  B T H W heads d k mode   plan fields and the host gather map
 *   c_caller attn  B T H W heads d k mode out.bin
 *                  bf16 forward on the device; q, k, v from an integer hash
 *                  (tensor t, element i): ((i * 2654435761 + t * 40503) mod 2^32
 *                  >> 8) / 2^24 - 0.5, exact in fp32 and bf16-rounded (nearest
 *                  even); writes the bf16 output to out.bin
 *   c_caller attn8 B T H W heads d k mode out.bin
 *                  the same inputs quantized per tensor to e4m3 on the
 *                  device (skiparse_quant_fp8, maximum 448), then the e4m3
 *                  forward; writes the bf16 output to out.bin
 *
 * Prints "error <code> <message>" and exits 1 on a library error.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "skiparse.h"

static int check(int code) {
  if (code != SKIPARSE_OK) {
    printf("error %d %s\n", code, skiparse_last_error());
    exit(1);
  }
  return code;
}

static uint16_t to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);   /* round to nearest even (finite inputs) */
  return (uint16_t)(u >> 16);
}

static float input_value(int t, uint64_t i) {
  const uint32_t h = (uint32_t)(i * 2654435761u + (uint32_t)t * 40503u);
  return (float)(h >> 8) / 16777216.0f - 0.5f;
}

int main(int argc, char** argv) {
  if (argc < 10) {
    fprintf(stderr, "usage: c_caller plan|attn|attn8 B T H W heads d k mode [out.bin]\n");
    return 2;
  }
  int v[8];
  for (int i = 0; i < 8; ++i) v[i] = atoi(argv[2 + i]);
  if (skiparse_abi_version() != SKIPARSE_ABI_VERSION) {
    printf("error abi\n");
    return 1;
  }
  skiparse_plan p;
  check(skiparse_plan_init(&p, v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7]));
  if (strcmp(argv[1], "plan") == 0) {
    printf("plan %d %d %d %d %d %lld %lld\n", p.Hp, p.Wp, p.sub_h, p.sub_w, p.n_sub, (long long)p.sub_len_padded,
           (long long)p.pairs);
    const size_t n = (size_t)p.n_sub * (size_t)p.sub_len_padded;
    int32_t* map = (int32_t*)malloc(n * sizeof(int32_t));
    check(skiparse_plan_index_map(&p, map));
    printf("map");
    for (size_t i = 0; i < n; ++i) printf(" %d", map[i]);
    printf("\n");
    free(map);
    /* an invalid call reports an error and leaves a message */
    const int bad = skiparse_plan_init(&p, 1, 1, 1, 1, 1, 64, 0, 0);
    printf("bad %d %s\n", bad, skiparse_last_error()[0] ? "message" : "none");
    return 0;
  }
  const int fp8 = strcmp(argv[1], "attn8") == 0;
  if ((strcmp(argv[1], "attn") == 0 || fp8) && argc >= 11) {
    const size_t numel = (size_t)v[0] * v[1] * v[2] * v[3] * v[4] * v[5];
    uint16_t* host = (uint16_t*)malloc(numel * 2);
    void* dev[4];
    for (int t = 0; t < 4; ++t) {
      if (hipMalloc(&dev[t], numel * 2) != hipSuccess) {
        printf("error hipMalloc\n");
        return 1;
      }
    }
    for (int t = 0; t < 3; ++t) {
      for (size_t i = 0; i < numel; ++i) host[i] = to_bf16(input_value(t, i));
      if (hipMemcpy(dev[t], host, numel * 2, hipMemcpyHostToDevice) != hipSuccess) {
        printf("error hipMemcpy\n");
        return 1;
      }
    }
    if (fp8) {
      void* codes[3];
      float* scales = NULL;
      void* ws = NULL;
      const size_t wsb = skiparse_quant_fp8_workspace_bytes((int64_t)numel);
      if (hipMalloc((void**)&scales, 6 * sizeof(float)) != hipSuccess || hipMalloc(&ws, wsb) != hipSuccess) {
        printf("error hipMalloc\n");
        return 1;
      }
      for (int t = 0; t < 3; ++t) {
        if (hipMalloc(&codes[t], numel) != hipSuccess) {
          printf("error hipMalloc\n");
          return 1;
        }
        check(skiparse_quant_fp8(dev[t], SKIPARSE_BF16, (int64_t)numel, (uint8_t*)codes[t], scales + 2 * t, 448.0f,
                                 1e-12f, ws, wsb, NULL));
      }
      check(skiparse_attn_fwd(&p, SKIPARSE_FP8_E4M3, codes[0], codes[1], codes[2], dev[3], 0.0f, scales, 0, 0,
                              NULL));
      if (hipDeviceSynchronize() != hipSuccess) {
        printf("error hip\n");
        return 1;
      }
      for (int t = 0; t < 3; ++t) hipFree(codes[t]);
      hipFree(scales);
      hipFree(ws);
    } else {
      check(skiparse_attn_fwd(&p, SKIPARSE_BF16, dev[0], dev[1], dev[2], dev[3], 0.0f, NULL, 0, 0, NULL));
    }
    if (hipDeviceSynchronize() != hipSuccess || hipMemcpy(host, dev[3], numel * 2, hipMemcpyDeviceToHost) != hipSuccess) {
      printf("error hip\n");
      return 1;
    }
    FILE* f = fopen(argv[10], "wb");
    if (!f || fwrite(host, 2, numel, f) != numel) {
      printf("error write\n");
      return 1;
    }
    fclose(f);
    for (int t = 0; t < 4; ++t) hipFree(dev[t]);
    free(host);
    printf("attn ok %zu\n", numel);
    return 0;
  }
  fprintf(stderr, "unknown command %s\n", argv[1]);
  return 2;
}
