/* Drives every entry point of include/mla.h through its validation paths
 * (NULL, misaligned and out-of-range arguments, invalid shapes, extreme
 * sizes) and through to the launch for valid arguments, in a build whose
 * host code carries AddressSanitizer and UndefinedBehaviorSanitizer. The
 * launchers are stubs that fail, so nothing runs on a device: valid calls
 * return MLA_ERR_HIP. Exit status 0 iff every status is the expected one
 * (the sanitizers abort on the first report). */
#include <limits.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../../include/mla.h"

static int failures = 0;

#define EXPECT(expr, want)                                                                         \
  do {                                                                                             \
    const long got_ = (long)(expr);                                                                \
    if (got_ != (long)(want)) {                                                                    \
      printf("FAIL line %d: %s -> %ld, expected %ld\n", __LINE__, #expr, got_, (long)(want));     \
      ++failures;                                                                                  \
    }                                                                                              \
  } while (0)

static mla_shape wan(void) {
  mla_shape s;
  memset(&s, 0, sizeof s);
  s.batch = 1;
  s.hidden = 1536;
  s.n_heads = 12;
  s.d_head = 128;
  s.d_c = 192;
  s.d_rope = 32;
  s.d_rope_t = 8;
  s.d_rope_y = 12;
  s.d_rope_x = 12;
  s.grid_y = 30;
  s.grid_x = 52;
  s.window_frames = 21;
  s.dtype = MLA_BF16;
  s.rope_base = 10000.f;
  s.softmax_scale = 0.f;
  return s;
}

int main(void) {
  void* p = (void*)(uintptr_t)0x100000; /* aligned, never dereferenced */
  void* odd = (void*)(uintptr_t)0x100008;
  float* tab = (float*)p;
  int32_t* sf = (int32_t*)p;
  mla_shape s = wan();
  const size_t big = (size_t)1 << 40;

  EXPECT(mla_abi_version(), MLA_ABI_VERSION);
  for (int c = -3; c < 12; ++c) EXPECT(mla_status_string(c) != NULL, 1);
  EXPECT(mla_shape_check(NULL), MLA_ERR_NULL);
  EXPECT(mla_shape_check(&s), MLA_OK);

  /* shape validation: each field out of range */
  {
    mla_shape t;
    t = s; t.dtype = 7; EXPECT(mla_shape_check(&t), MLA_ERR_DTYPE);
    t = s; t.batch = 0; EXPECT(mla_shape_check(&t), MLA_ERR_SHAPE);
    t = s; t.batch = INT_MAX; EXPECT(mla_shape_check(&t), MLA_ERR_SHAPE);
    t = s; t.hidden = 12; EXPECT(mla_shape_check(&t), MLA_ERR_SHAPE);
    t = s; t.d_head = 264; EXPECT(mla_shape_check(&t), MLA_ERR_SHAPE);
    t = s; t.window_frames = 65; EXPECT(mla_shape_check(&t), MLA_ERR_SHAPE);
    t = s; t.d_rope_t = 7; EXPECT(mla_shape_check(&t), MLA_ERR_SHAPE);
    t = s; t.d_rope_x = 14; EXPECT(mla_shape_check(&t), MLA_ERR_SHAPE);
    t = s; t.grid_y = INT_MAX; t.grid_x = INT_MAX; EXPECT(mla_shape_check(&t), MLA_ERR_SHAPE);
    t = s; t.grid_y = 2048; t.grid_x = 2048; EXPECT(mla_shape_check(&t), MLA_ERR_SHAPE);
    t = s; t.rope_base = -1.f; EXPECT(mla_shape_check(&t), MLA_ERR_SHAPE);
    t = s; t.d_rope_t = INT_MAX - 1; t.d_rope_y = INT_MAX - 1; EXPECT(mla_shape_check(&t), MLA_ERR_SHAPE);
    t = s; t.d_c = INT_MAX; EXPECT(mla_shape_check(&t), MLA_ERR_SHAPE);
    t = s; t.n_heads = INT_MAX; EXPECT(mla_shape_check(&t), MLA_OK);
    EXPECT(mla_chunk_attend_workspace_bytes(&t, 3), 0);
    EXPECT(mla_query_project(&t, 576, p, 3, p, p, p, p, p, p, NULL), MLA_ERR_SHAPE);
    t = s; t.d_c = 96; EXPECT(mla_shape_check(&t), MLA_ERR_UNSUPPORTED);
    EXPECT(mla_qabs_dim(&t), 0);
    EXPECT(mla_rope3d_table_floats(&t, 21), 0);
    EXPECT(mla_chunk_attend_workspace_bytes(&t, 3), 0);
  }

  /* host queries at valid and extreme sizes */
  EXPECT(mla_qabs_dim(&s), 224);
  EXPECT(mla_rope3d_table_floats(&s, 21) > 0, 1);
  EXPECT(mla_rope3d_table_floats(&s, 0), 0);
  EXPECT(mla_rope3d_table_floats(&s, -5), 0);
  EXPECT(mla_flash_workspace_bytes(&s, 3, 0) > 0, 1);
  EXPECT(mla_flash_workspace_bytes(&s, 3, 16) > 0, 1);
  EXPECT(mla_flash_workspace_bytes(&s, 3, 17), 0);
  EXPECT(mla_flash_workspace_bytes(&s, 0, 0), 0);
  EXPECT(mla_chunk_attend_workspace_bytes(&s, 3) > 0, 1);
  EXPECT(mla_chunk_attend_workspace_bytes(&s, INT_MAX), 0);
  EXPECT(mla_chunk_attend_heads_workspace_bytes(&s, 3) > 0, 1);
  {
    mla_shape t = s;
    t.batch = 4096;
    t.window_frames = 64;
    (void)mla_chunk_attend_workspace_bytes(&t, 64); /* large but finite sizes */
    (void)mla_chunk_attend_heads_workspace_bytes(&t, 64);
    t.dtype = MLA_F32;
    EXPECT(mla_chunk_attend_heads_workspace_bytes(&t, 3), 0);
  }

  /* RoPE tables */
  EXPECT(mla_rope3d_tables(&s, 0, 21, NULL, NULL), MLA_ERR_NULL);
  EXPECT(mla_rope3d_tables(&s, 0, 21, (float*)odd, NULL), MLA_ERR_ALIGN);
  EXPECT(mla_rope3d_tables(&s, -1, 21, tab, NULL), MLA_ERR_RANGE);
  EXPECT(mla_rope3d_tables(&s, INT_MAX, 21, tab, NULL), MLA_ERR_RANGE);
  EXPECT(mla_rope3d_tables(&s, 0, 21, tab, NULL), MLA_ERR_HIP);

  /* cache write */
  EXPECT(mla_cache_write(&s, NULL, p, p, 0, 3, p, sf, NULL), MLA_ERR_NULL);
  EXPECT(mla_cache_write(&s, odd, p, p, 0, 3, p, sf, NULL), MLA_ERR_ALIGN);
  EXPECT(mla_cache_write(&s, p, p, p, 0, 22, p, sf, NULL), MLA_ERR_RANGE);
  EXPECT(mla_cache_write(&s, p, p, p, 0, 0, p, sf, NULL), MLA_ERR_RANGE);
  EXPECT(mla_cache_write(&s, p, p, p, -1, 3, p, sf, NULL), MLA_ERR_RANGE);
  EXPECT(mla_cache_write(&s, p, p, p, INT_MAX, 3, p, sf, NULL), MLA_ERR_RANGE);
  EXPECT(mla_cache_write(&s, p, p, p, 18, 3, p, sf, NULL), MLA_ERR_HIP);

  /* absorb, flash, up-projection */
  EXPECT(mla_absorb_q(&s, p, p, 30, 3, p, tab, 0, 21, p, NULL), MLA_ERR_RANGE);
  EXPECT(mla_absorb_q(&s, p, p, 0, INT_MAX, p, tab, 0, 21, p, NULL), MLA_ERR_SHAPE);
  EXPECT(mla_absorb_q(&s, p, p, 18, 3, p, tab, 0, 21, p, NULL), MLA_ERR_HIP);
  EXPECT(mla_flash_attend(&s, p, 3, p, sf, tab, 0, 21, p, 0, p, 16, NULL), MLA_ERR_WORKSPACE);
  EXPECT(mla_flash_attend(&s, p, 3, p, sf, tab, 0, 21, p, -1, p, big, NULL), MLA_ERR_RANGE);
  EXPECT(mla_flash_attend(&s, p, 3, p, sf, tab, 0, 21, p, 0, p, big, NULL), MLA_ERR_HIP);
  EXPECT(mla_flash_attend(&s, p, 3, p, sf, tab, 0, 21, p, 3, p, big, NULL), MLA_ERR_HIP);
  EXPECT(mla_up_v(&s, p, 3, NULL, p, NULL), MLA_ERR_NULL);
  EXPECT(mla_up_v(&s, p, 3, p, p, NULL), MLA_ERR_HIP);

  /* whole attention side, its variants and the per-head form */
  EXPECT(mla_chunk_attend(&s, p, p, 18, 3, p, p, p, sf, tab, 0, 21, p, p, 16, NULL), MLA_ERR_WORKSPACE);
  EXPECT(mla_chunk_attend(&s, p, p, 18, 3, p, p, p, sf, tab, 20, 21, p, p, big, NULL), MLA_ERR_RANGE);
  EXPECT(mla_chunk_attend(&s, p, p, 18, 3, p, p, p, sf, tab, 0, 21, p, p, big, NULL), MLA_ERR_HIP);
  EXPECT(mla_chunk_attend_frame_causal(&s, p, p, 18, 3, p, p, p, sf, tab, 0, 21, p, p, big, NULL), MLA_ERR_HIP);
  EXPECT(mla_chunk_attend_heads(&s, p, p, 18, 3, p, p, p, sf, tab, 0, 21, p, p, 16, NULL), MLA_ERR_WORKSPACE);
  EXPECT(mla_chunk_attend_heads(&s, p, p, 18, 3, p, p, p, sf, tab, 0, 21, p, p, big, NULL), MLA_ERR_HIP);
  EXPECT(mla_chunk_attend_latent_frame_causal(&s, p, p, 18, 3, p, p, p, sf, tab, 0, 21, p, p, 16, NULL),
         MLA_ERR_WORKSPACE);
  EXPECT(mla_chunk_attend_latent_frame_causal(&s, p, p, 18, 3, p, p, p, sf, tab, 0, 21, p, p, big, NULL), MLA_ERR_HIP);
  EXPECT(mla_chunk_attend_heads_frame_causal(&s, p, p, 18, 3, p, p, p, sf, tab, 0, 21, p, p, 16, NULL),
         MLA_ERR_WORKSPACE);
  EXPECT(mla_chunk_attend_heads_frame_causal(&s, p, p, 18, 3, p, p, p, sf, tab, 0, 21, p, p, big, NULL), MLA_ERR_HIP);
  {
    /* several streams: both plans deal whole row blocks in rounds, also
       with the row-block classes of the frame-causal mask */
    mla_shape t = s;
    t.batch = 8;
    EXPECT(mla_chunk_attend_latent_frame_causal(&t, p, p, 18, 3, p, p, p, sf, tab, 0, 21, p, p, big, NULL), MLA_ERR_HIP);
    EXPECT(mla_chunk_attend_heads_frame_causal(&t, p, p, 18, 3, p, p, p, sf, tab, 0, 21, p, p, big, NULL), MLA_ERR_HIP);
    EXPECT(mla_chunk_attend_frame_causal(&t, p, p, 18, 3, p, p, p, sf, tab, 0, 21, p, p, big, NULL), MLA_ERR_HIP);
    EXPECT(mla_chunk_attend(&t, p, p, 18, 3, p, p, p, sf, tab, 0, 21, p, p, big, NULL), MLA_ERR_HIP);
    /* a 64-frame chunk over a 64-frame window: the most row-block classes a plan builds */
    t.window_frames = 64;
    EXPECT(mla_chunk_attend_heads_frame_causal(&t, p, p, 0, 64, p, p, p, sf, tab, 0, 64, p, p, big, NULL), MLA_ERR_HIP);
    EXPECT(mla_chunk_attend_latent_frame_causal(&t, p, p, 0, 64, p, p, p, sf, tab, 0, 64, p, p, big, NULL), MLA_ERR_HIP);
  }

  /* query path and output projection */
  EXPECT(mla_query_project(&s, 576, p, 3, p, p, NULL, p, p, p, NULL), MLA_ERR_NULL);
  EXPECT(mla_query_project(&s, 576, p, 3, p, p, p, odd, p, p, NULL), MLA_ERR_ALIGN);
  EXPECT(mla_query_project(&s, 572, p, 3, p, p, p, p, p, p, NULL), MLA_ERR_SHAPE);
  EXPECT(mla_query_project(&s, INT_MAX, p, 3, p, p, p, p, p, p, NULL), MLA_ERR_SHAPE);
  EXPECT(mla_query_project(&s, 576, p, INT_MAX, p, p, p, p, p, p, NULL), MLA_ERR_SHAPE);
  EXPECT(mla_query_project(&s, 576, p, 3, p, p, p, p, p, p, NULL), MLA_ERR_HIP);
  EXPECT(mla_output_project(&s, p, 0, p, p, NULL), MLA_ERR_RANGE);
  {
    mla_shape t = s; /* 2^29 rows: fine for 1536 outputs, too many tiles for 65536 */
    t.batch = 1 << 13;
    t.grid_y = 64;
    t.grid_x = 64;
    t.window_frames = 1;
    EXPECT(mla_shape_check(&t), MLA_OK);
    EXPECT(mla_output_project(&t, p, 16, p, p, NULL), MLA_ERR_HIP);
    EXPECT(mla_query_project(&t, 65536, p, 16, p, p, p, p, p, p, NULL), MLA_ERR_SHAPE);
  }
  EXPECT(mla_output_project(&s, p, 3, p, p, NULL), MLA_ERR_HIP);

  /* absorbed query path */
  EXPECT(mla_query_absorb_weights(&s, 576, p, p, NULL, p, NULL), MLA_ERR_NULL);
  EXPECT(mla_query_absorb_weights(&s, 576, p, p, p, odd, NULL), MLA_ERR_ALIGN);
  EXPECT(mla_query_absorb_weights(&s, 570, p, p, p, p, NULL), MLA_ERR_SHAPE);
  EXPECT(mla_query_absorb_weights(&s, 576, p, p, p, p, NULL), MLA_ERR_HIP);
  EXPECT(mla_query_project_absorbed(&s, 576, p, 18, 3, p, p, tab, 0, 21, p, NULL, NULL), MLA_ERR_NULL);
  EXPECT(mla_query_project_absorbed(&s, 576, p, 18, 3, p, p, tab, 19, 21, p, p, NULL), MLA_ERR_RANGE);
  EXPECT(mla_query_project_absorbed(&s, 576, p, 18, 0, p, p, tab, 0, 21, p, p, NULL), MLA_ERR_RANGE);
  EXPECT(mla_query_project_absorbed(&s, 576, p, 18, 3, p, p, tab, 0, 21, p, p, NULL), MLA_ERR_HIP);

  /* whole layer */
  {
    mla_layer_weights lw = {p, p, p, p, p, p, p, p, NULL};
    const size_t need = mla_layer_step_workspace_bytes(&s, 576, 3);
    EXPECT(need > mla_chunk_attend_workspace_bytes(&s, 3), 1);
    EXPECT(mla_layer_step_workspace_bytes(&s, 572, 3), 0);
    EXPECT(mla_layer_step_workspace_bytes(&s, 576, 0), 0);
    EXPECT(mla_layer_step(&s, 576, NULL, p, 18, 3, p, sf, tab, 0, 21, 0, p, p, need, NULL), MLA_ERR_NULL);
    EXPECT(mla_layer_step(&s, 576, &lw, p, 18, 3, p, sf, tab, 0, 21, 0, p, p, need - 1, NULL), MLA_ERR_WORKSPACE);
    EXPECT(mla_layer_step(&s, 576, &lw, p, 18, 22, p, sf, tab, 0, 40, 0, p, p, big, NULL), MLA_ERR_RANGE);
    EXPECT(mla_layer_step(&s, 576, &lw, p, 18, 3, p, sf, tab, 19, 21, 0, p, p, need, NULL), MLA_ERR_RANGE);
    lw.w_o = NULL;
    EXPECT(mla_layer_step(&s, 576, &lw, p, 18, 3, p, sf, tab, 0, 21, 0, p, p, need, NULL), MLA_ERR_NULL);
    lw.w_o = odd;
    EXPECT(mla_layer_step(&s, 576, &lw, p, 18, 3, p, sf, tab, 0, 21, 1, p, p, need, NULL), MLA_ERR_ALIGN);
    lw.w_o = p;
    EXPECT(mla_layer_step(&s, 576, &lw, p, 18, 3, p, sf, tab, 0, 21, 1, p, p, need, NULL), MLA_ERR_HIP);
    lw.w_qabs = p; /* fused query path */
    lw.w_uq = lw.w_qr = lw.w_uk = NULL; /* not read */
    EXPECT(mla_layer_step(&s, 576, &lw, p, 18, 3, p, sf, tab, 0, 21, 0, p, p, need - 1, NULL), MLA_ERR_WORKSPACE);
    EXPECT(mla_layer_step(&s, 576, &lw, p, 18, 3, p, sf, tab, 19, 21, 0, p, p, need, NULL), MLA_ERR_RANGE);
    EXPECT(mla_layer_step(&s, 576, &lw, p, 18, 3, p, sf, tab, 0, 21, 1, p, p, need, NULL), MLA_ERR_HIP);
  }

  printf("%s: %d unexpected statuses\n", failures ? "FAILED" : "ok", failures);
  return failures != 0;
}
