/* A chunk step driven from plain C (gcc) through include/mla.h alone: RoPE tables, a
 * prefill of three frames, the cache write of a two-frame chunk, the
 * attention, on a small grid with the Wan2.1-1.3B head shapes. Inputs are
 * bf16 bit patterns from a fixed linear congruential generator (the Python
 * side of the test draws the same bits); the output is written raw to the
 * file named by argv[1]. Exit status 0 on success. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "../../include/mla.h"

static uint64_t lcg_state = 0x2545F4914F6CDD1Dull;

/* bf16 bits of a value in +-[2^-7, 2): random sign, exponent 120..127, mantissa */
static uint16_t next_bf16(void) {
  lcg_state = lcg_state * 6364136223846793005ull + 1442695040888963407ull;
  const uint32_t r = (uint32_t)(lcg_state >> 33);
  const uint32_t sign = r & 1u, expo = 120u + ((r >> 1) & 7u), mant = (r >> 4) & 0x7fu;
  return (uint16_t)((sign << 15) | (expo << 7) | mant);
}

static void* device_fill(size_t n) {
  uint16_t* h = (uint16_t*)malloc(n * 2);
  for (size_t i = 0; i < n; ++i) h[i] = next_bf16();
  void* d = NULL;
  if (hipMalloc(&d, n * 2) != hipSuccess || hipMemcpy(d, h, n * 2, hipMemcpyHostToDevice) != hipSuccess) {
    free(h);
    return NULL;
  }
  free(h);
  return d;
}

#define CHECK(x)                                                             \
  do {                                                                       \
    const int st_ = (int)(x);                                                \
    if (st_ != 0) {                                                          \
      fprintf(stderr, "%s failed: %d (%s)\n", #x, st_, mla_status_string(st_)); \
      return 1;                                                              \
    }                                                                        \
  } while (0)

int main(int argc, char** argv) {
  if (argc < 2) return 2;
  mla_shape s = {1, 1536, 12, 128, 192, 32, 8, 12, 12, 6, 11, 5, MLA_BF16, 10000.f, 0.f};
  const int T = s.grid_y * s.grid_x, W = s.window_frames, H = s.n_heads;
  const int chunk_first = 3, chunk_n = 2, n_t = 16;
  CHECK(mla_shape_check(&s));
  /* inputs in a fixed order: weights, then tokens of frames 0..4, then queries */
  void* w_dkv = device_fill((size_t)s.d_c * s.hidden);
  void* w_kr = device_fill((size_t)s.d_rope * s.hidden);
  void* w_uk = device_fill((size_t)H * s.d_head * s.d_c);
  void* w_uv = device_fill((size_t)H * s.d_head * s.d_c);
  void* x_pre = device_fill((size_t)chunk_first * T * s.hidden);
  void* x_chunk = device_fill((size_t)chunk_n * T * s.hidden);
  void* q_nope = device_fill((size_t)chunk_n * T * H * s.d_head);
  void* q_r = device_fill((size_t)chunk_n * T * H * s.d_rope);
  if (!w_dkv || !w_kr || !w_uk || !w_uv || !x_pre || !x_chunk || !q_nope || !q_r) return 3;

  void *cache = NULL, *slot = NULL, *tables = NULL, *out = NULL, *ws = NULL;
  const size_t cache_bytes = (size_t)W * T * (s.d_c + s.d_rope) * 2;
  const size_t out_bytes = (size_t)chunk_n * T * H * s.d_head * 2;
  const size_t ws_bytes = mla_chunk_attend_workspace_bytes(&s, chunk_n);
  const size_t tab_bytes = mla_rope3d_table_floats(&s, n_t) * sizeof(float);
  if (ws_bytes == 0 || tab_bytes == 0) return 4;
  if (hipMalloc(&cache, cache_bytes) || hipMalloc(&slot, W * sizeof(int32_t)) || hipMalloc(&tables, tab_bytes) ||
      hipMalloc(&out, out_bytes) || hipMalloc(&ws, ws_bytes))
    return 5;
  if (hipMemset(cache, 0, cache_bytes) || hipMemset(slot, 0xff, W * sizeof(int32_t))) return 6; /* slot_frame = -1 */

  CHECK(mla_rope3d_tables(&s, 0, n_t, (float*)tables, NULL));
  CHECK(mla_cache_write(&s, x_pre, w_dkv, w_kr, 0, chunk_first, cache, (int32_t*)slot, NULL));
  CHECK(mla_cache_write(&s, x_chunk, w_dkv, w_kr, chunk_first, chunk_n, cache, (int32_t*)slot, NULL));
  CHECK(mla_chunk_attend(&s, q_nope, q_r, chunk_first, chunk_n, w_uk, w_uv, cache, (const int32_t*)slot,
                         (const float*)tables, 0, n_t, out, ws, ws_bytes, NULL));
  if (hipDeviceSynchronize() != hipSuccess) return 7;

  void* h = malloc(out_bytes);
  if (hipMemcpy(h, out, out_bytes, hipMemcpyDeviceToHost) != hipSuccess) return 8;
  FILE* f = fopen(argv[1], "wb");
  if (!f || fwrite(h, 1, out_bytes, f) != out_bytes) return 9;
  fclose(f);
  free(h);
  printf("chunk step from C: %zu output bytes\n", out_bytes);
  return 0;
}
