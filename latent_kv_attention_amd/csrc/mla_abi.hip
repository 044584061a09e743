// C ABI layer: argument validation, workspace sizing and kernel dispatch.
// Everything here runs on the host; no entry point allocates memory, and no
// C++ exception leaves this file.
#include <math.h>
#include <stdint.h>

#include "../../include/mla.h"
#include "abi_internal.hpp"
#include "mla_internal.hpp"

#define MLA_API extern "C" __attribute__((visibility("default")))

namespace {

using mla::RopeLayout;

constexpr int kMaxWindow = 64;
constexpr int kMaxHeadDim = 256;
constexpr int kMaxSplits = 16;
constexpr int kAssumedCUs = 256;  // MI355X; only steers the automatic split choice

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t elt_size(const mla_shape* s) { return s->dtype == MLA_BF16 ? 2 : 4; }

// latent widths with kernel instantiations: the Wan2.1 split (192, 32), a
// smaller latent (128, 32), the same 224 scalars split (160, 64), a larger
// latent (192, 64), and the small test widths (16, 8)
bool latent_supported(int d_c, int d_rope) {
  return (d_c == 192 && d_rope == 32) || (d_c == 128 && d_rope == 32) || (d_c == 160 && d_rope == 64) ||
         (d_c == 192 && d_rope == 64) || (d_c == 16 && d_rope == 8);
}

mla_status check_shape(const mla_shape* s) {
  if (!s) return MLA_ERR_NULL;
  if (s->dtype != MLA_BF16 && s->dtype != MLA_F32) return MLA_ERR_DTYPE;
  if (s->batch < 1 || s->n_heads < 1 || s->grid_y < 1 || s->grid_x < 1) return MLA_ERR_SHAPE;
  if (s->hidden < 8 || s->hidden % 8 != 0) return MLA_ERR_SHAPE;
  if (s->d_head < 8 || s->d_head % 8 != 0 || s->d_head > kMaxHeadDim) return MLA_ERR_SHAPE;
  if (s->window_frames < 1 || s->window_frames > kMaxWindow) return MLA_ERR_SHAPE;
  if (s->d_rope_t < 0 || s->d_rope_y < 0 || s->d_rope_x < 0) return MLA_ERR_SHAPE;
  if (s->d_rope_t % 2 || s->d_rope_y % 2 || s->d_rope_x % 2) return MLA_ERR_SHAPE;
  if ((int64_t)s->d_rope_t + s->d_rope_y + s->d_rope_x != s->d_rope) return MLA_ERR_SHAPE;
  if (s->d_c < 1 || s->d_rope < 1) return MLA_ERR_SHAPE;
  if (!(s->rope_base > 0.f) || !isfinite(s->rope_base)) return MLA_ERR_SHAPE;
  if (!isfinite(s->softmax_scale)) return MLA_ERR_SHAPE;
  // (each product below is bounded by the checks before it, so none overflows)
  const int64_t T = (int64_t)s->grid_y * s->grid_x;
  // the attention kernel splits key indices with a float reciprocal (exact
  // below 2^22 keys per window)
  if (T > mla::kMaxWindowKeys || T * s->window_frames > mla::kMaxWindowKeys) return MLA_ERR_SHAPE;
  if (s->d_c > (1 << 16) || s->d_rope > (1 << 16)) return MLA_ERR_SHAPE;
  // per-stream cache element offsets are 32-bit inside the kernels
  if (T * s->window_frames * (s->d_c + s->d_rope) > INT32_MAX) return MLA_ERR_SHAPE;
  if ((int64_t)s->batch * s->window_frames * T * (s->d_c + s->d_rope) > INT64_C(1) << 40) return MLA_ERR_SHAPE;
  if (!latent_supported(s->d_c, s->d_rope)) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

int64_t tokens_per_frame(const mla_shape* s) { return (int64_t)s->grid_y * s->grid_x; }

int qabs_dim(const mla_shape* s) { return (s->d_c + s->d_rope + 31) / 32 * 32; }

float scale_log2(const mla_shape* s) {
  const double scale = s->softmax_scale > 0.f ? (double)s->softmax_scale : 1.0 / sqrt((double)(s->d_head + s->d_rope));
  return (float)(scale * 1.4426950408889634);  // log2(e)
}

RopeLayout rope_layout(const mla_shape* s, int t_first, int n_t) {
  RopeLayout rl;
  rl.d_t = s->d_rope_t;
  rl.d_y = s->d_rope_y;
  rl.d_x = s->d_rope_x;
  rl.t_first = t_first;
  rl.n_t = n_t;
  rl.off_ct = 0;
  rl.off_st = rl.off_ct + n_t * (rl.d_t / 2);
  rl.off_cy = rl.off_st + n_t * (rl.d_t / 2);
  rl.off_sy = rl.off_cy + s->grid_y * (rl.d_y / 2);
  rl.off_cx = rl.off_sy + s->grid_y * (rl.d_y / 2);
  rl.off_sx = rl.off_cx + s->grid_x * (rl.d_x / 2);
  return rl;
}

size_t table_floats(const mla_shape* s, int n_t) {
  return 2 * ((size_t)n_t * (s->d_rope_t / 2) + (size_t)s->grid_y * (s->d_rope_y / 2) +
              (size_t)s->grid_x * (s->d_rope_x / 2));
}

size_t round256(size_t n) { return (n + 255) / 256 * 256; }

int flash_rows_per_block(const mla_shape* s) { return s->dtype == MLA_BF16 ? 256 : 128; }
int flash_tile_keys(const mla_shape* s) { return s->dtype == MLA_BF16 ? 128 : 32; }

// Compute units of the current device (the automatic work split uses one
// work-group per compute unit); falls back to the MI355X count.
int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return kAssumedCUs;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
    return kAssumedCUs;
  return n;
}

// Work split of the attention kernel: `grid` work-groups share `units`
// (row block, key tile) pairs evenly. kv_splits = s > 0 gives every row
// block s equal key ranges (s = 1: one work-group per row block);
// kv_splits = 0 uses one work-group per compute unit, and where there are
// at least as many row blocks as work-groups (several streams) deals the
// first whole multiple of `grid` row blocks out whole, in rounds, and shares
// the units after them. (Under the frame-causal mask the row blocks of a
// round differ in units by the window frames their rows may not see, at
// most the chunk's length in frames.)
struct FlashPlan {
  int n_rb, nt_max;
  int64_t units;
  int grid;
  int64_t rb_whole;  // row blocks dealt whole in rounds (a multiple of grid)
  int64_t u_rest;    // first unit after them
  int grid_rest;     // work-groups sharing the units from u_rest on
  bool split;        // some row block is shared by several work-groups
  mla::UnitClasses classes;
};

// With the frame-causal mask and the automatic split, a row block's units
// cover only the keys its rows may see: with keys in frame order, the frames
// up to its last row's, W - (q_n_frames - 1 - k) frames of a full window for
// a row block whose last row is a query of chunk frame k. Without the mask
// (or with fixed key splits) every row block has the nt_max tiles of a full
// window.
FlashPlan flash_plan(const mla_shape* s, int q_n_frames, int kv_splits, bool causal = false) {
  FlashPlan f;
  const int64_t T = tokens_per_frame(s);
  const int64_t Mb = (int64_t)q_n_frames * T * s->n_heads;
  const int rpb = flash_rows_per_block(s), tk = flash_tile_keys(s);
  f.n_rb = (int)((Mb + rpb - 1) / rpb);
  f.nt_max = (int)((s->window_frames * T + tk - 1) / tk);
  mla::UnitClasses& c = f.classes;
  c = mla::UnitClasses{};
  if (causal && kv_splits == 0 && q_n_frames <= mla::kMaxUnitClasses) {
    const int64_t rows_per_frame = T * s->n_heads;
    int64_t u = 0;
    c.n = 0;
    for (int k = 0; k < q_n_frames; ++k) {
      // row blocks whose last row lies in chunk frame k
      const int64_t end = k + 1 < q_n_frames ? ((k + 1) * rows_per_frame) / rpb : f.n_rb;
      const int64_t start = c.n == 0 ? 0 : c.rb_end[c.n - 1];
      if (end <= start) continue;
      const int64_t frames = (int64_t)s->window_frames - (q_n_frames - 1 - k);
      const int nt = (int)(frames < 1 ? 1 : (frames * T + tk - 1) / tk);
      c.rb_end[c.n] = (int)end;
      c.nt[c.n] = nt;
      c.u0[c.n] = u;
      u += (end - start) * nt;
      ++c.n;
    }
    c.per_stream = u;
  } else {
    c.n = 1;
    c.rb_end[0] = f.n_rb;
    c.nt[0] = f.nt_max;
    c.u0[0] = 0;
    c.per_stream = (int64_t)f.n_rb * f.nt_max;
  }
  f.units = (int64_t)s->batch * c.per_stream;
  const int64_t row_blocks = (int64_t)s->batch * f.n_rb;
  int64_t g = kv_splits > 0 ? row_blocks * kv_splits : device_cus();
  if (g > f.units) g = f.units;
  // a row block meets fewer than units/(units/G) + 1 ranges: keep that <= kMaxMergePieces
  if (g > (mla::kMaxMergePieces - 1) * row_blocks) g = (mla::kMaxMergePieces - 1) * row_blocks;
  if (g < 1) g = 1;
  if (g > (INT64_C(1) << 23)) g = INT64_C(1) << 23;  // rejected by flash_plan_ok
  f.grid = (int)g;
  f.rb_whole = 0;
  if (kv_splits == 0 && row_blocks >= g) f.rb_whole = row_blocks / g * g;
  long long u_rest;
  int nt_unused;
  mla::row_block_units(c, f.n_rb, f.rb_whole, u_rest, nt_unused);  // (rb_whole = all row blocks: U)
  f.u_rest = u_rest;
  const int64_t rest = f.units - f.u_rest;
  // the rest: at most kMaxMergePieces - 1 work-groups per remaining row block
  int64_t gr = g;
  if (f.rb_whole > 0) {
    const int64_t rb_rest = row_blocks - f.rb_whole;
    if (gr > (mla::kMaxMergePieces - 1) * rb_rest) gr = (mla::kMaxMergePieces - 1) * rb_rest;
    if (gr > rest) gr = rest;
  }
  f.grid_rest = (int)gr;
  f.split = c.n > 1 || (rest > 0 && !(rest % gr == 0 && (rest / gr) % f.nt_max == 0));
  return f;
}

// unit and work-group indices stay far from 64-bit overflow (g * units)
bool flash_plan_ok(const FlashPlan& f) {
  return f.units <= (INT64_C(1) << 40) && f.grid <= (1 << 22);
}

// Flash workspace: the fallback row list, the window's rotated kR (one row
// of d_rope elements per key) and, when row blocks are shared, two partial
// (output / sum in the cache's element type, reference and sum in float)
// slots per work-group.
struct FlashWs {
  size_t count, rows, krot, part_o, part_l, total;
};

FlashWs flash_ws_layout(const mla_shape* s, int q_n_frames, const FlashPlan& f) {
  const size_t rows = (size_t)s->batch * q_n_frames * tokens_per_frame(s) * s->n_heads;
  const size_t slots = f.split ? (size_t)f.grid * 2 * flash_rows_per_block(s) : 0;
  FlashWs w;
  w.count = 0;
  w.rows = w.count + 256;
  w.krot = w.rows + round256(rows * sizeof(int));
  w.part_o = w.krot + round256((size_t)s->batch * s->window_frames * tokens_per_frame(s) * s->d_rope * elt_size(s));
  w.part_l = w.part_o + round256(slots * s->d_c * elt_size(s));
  w.total = w.part_l + round256(slots * 2 * sizeof(float));
  return w;
}

// (covers both masks: the frame-causal plan may split row blocks where the
// plain one does not)
size_t flash_ws_bytes(const mla_shape* s, int q_n_frames, int kv_splits) {
  const size_t a = flash_ws_layout(s, q_n_frames, flash_plan(s, q_n_frames, kv_splits, false)).total;
  const size_t b = flash_ws_layout(s, q_n_frames, flash_plan(s, q_n_frames, kv_splits, true)).total;
  return a > b ? a : b;
}

mla_status from_hip(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_HIP; }

mla_status check_tables(const mla_shape* s, const float* tables, int t_first, int n_t) {
  (void)s;
  if (!tables) return MLA_ERR_NULL;
  if (!aligned16(tables)) return MLA_ERR_ALIGN;
  if (n_t < 1 || t_first < 0) return MLA_ERR_RANGE;
  return MLA_OK;
}

mla_status do_absorb(const mla_shape* s, const void* q_nope, const void* q_r, int q_frame_first, int q_n_frames,
                     const void* w_uk, const float* tables, int rope_t_first, int rope_n_t, void* q_abs,
                     hipStream_t st) {
  mla::AbsorbParams p;
  p.q_nope = q_nope;
  p.q_r = q_r;
  p.w_uk = w_uk;
  p.tables = tables;
  p.q_abs = q_abs;
  p.rl = rope_layout(s, rope_t_first, rope_n_t);
  p.n_q = (int)(q_n_frames * tokens_per_frame(s));
  p.rows = s->batch * p.n_q;
  p.H = s->n_heads;
  p.d_head = s->d_head;
  p.T = (int)tokens_per_frame(s);
  p.grid_x = s->grid_x;
  p.q_frame_first = q_frame_first;
  p.qscale = scale_log2(s);
  return from_hip(mla::launch_absorb_q(s->dtype, s->d_c, s->d_rope, p, st));
}

mla_status do_flash(const mla_shape* s, const void* q_abs, int q_n_frames, const void* cache,
                    const int32_t* slot_frame, const float* tables, int rope_t_first, int rope_n_t, void* o_lat,
                    int kv_splits, void* ws, hipStream_t st, bool frame_causal = false, int q_frame_first = 0) {
  const FlashPlan f = flash_plan(s, q_n_frames, kv_splits, frame_causal);
  mla::FlashParams p;
  p.q_abs = q_abs;
  p.cache = cache;
  p.slot_frame = slot_frame;
  p.tables = tables;
  p.o_lat = o_lat;
  const FlashWs w = flash_ws_layout(s, q_n_frames, f);
  char* base = (char*)ws;
  p.fallback_count = (int*)(base + w.count);
  p.fallback_rows = (int*)(base + w.rows);
  p.part_o = f.split ? (void*)(base + w.part_o) : nullptr;
  p.part_l = f.split ? (float*)(base + w.part_l) : nullptr;
  p.krot = base + w.krot;
  p.rl = rope_layout(s, rope_t_first, rope_n_t);
  p.Mb = (int)(q_n_frames * tokens_per_frame(s) * s->n_heads);
  p.W = s->window_frames;
  p.T = (int)tokens_per_frame(s);
  p.grid_y = s->grid_y;
  p.grid_x = s->grid_x;
  p.inv_T = 1.f / (float)p.T;
  p.inv_grid_x = 1.f / (float)s->grid_x;
  p.batch = s->batch;
  p.n_rb = f.n_rb;
  p.nt_max = f.nt_max;
  p.units = f.units;
  p.classes = f.classes;
  p.grid = f.grid;
  p.rb_whole = f.rb_whole;
  p.u_rest = f.u_rest;
  p.grid_rest = f.grid_rest;
  p.scale_log2 = scale_log2(s);
  p.rope_base = (double)s->rope_base;
  p.H = s->n_heads;
  p.q_frame_first = q_frame_first;
  return from_hip(mla::launch_flash(s->dtype, s->d_c, s->d_rope, p, f.split, frame_causal, st));
}

mla_status do_up_v(const mla_shape* s, const void* o_lat, int q_n_frames, const void* w_uv, void* out,
                   hipStream_t st) {
  mla::UpVParams p;
  p.o_lat = o_lat;
  p.w_uv = w_uv;
  p.out = out;
  p.rows = (int)(s->batch * q_n_frames * tokens_per_frame(s));
  p.H = s->n_heads;
  p.d_head = s->d_head;
  return from_hip(mla::launch_up_v(s->dtype, s->d_c, s->d_rope, p, st));
}

mla_status check_query_args(const mla_shape* s, int q_frame_first, int q_n_frames) {
  if (q_frame_first < 0 || q_n_frames < 1) return MLA_ERR_RANGE;
  const int64_t rows = (int64_t)s->batch * q_n_frames * tokens_per_frame(s) * s->n_heads;
  if (rows > INT32_MAX / 2) return MLA_ERR_SHAPE;
  return MLA_OK;
}

// Work split of the per-head attention kernel: (row block of 384 tokens of
// one (stream, head), key tile) units shared evenly by one work-group per
// compute unit, as for the latent form (whole row blocks in rounds where
// there are enough of them). Under the frame-causal mask the row blocks of a
// (stream, head) form classes by the chunk frame of their last token, each
// with the units of the window part its tokens may see.
FlashPlan heads_plan(const mla_shape* s, int q_n_frames, bool causal = false) {
  FlashPlan f;
  const int64_t T = tokens_per_frame(s);
  const int64_t nq = (int64_t)q_n_frames * T;
  const int tk = mla::heads_tile_keys(s->d_head, s->d_rope);
  const int rpb = mla::kHeadsRowsPerBlock;
  f.n_rb = (int)((nq + rpb - 1) / rpb);
  f.nt_max = (int)((s->window_frames * T + tk - 1) / tk);
  mla::UnitClasses& c = f.classes;
  c = mla::UnitClasses{};
  if (causal && q_n_frames <= mla::kMaxUnitClasses) {
    int64_t u = 0;
    c.n = 0;
    for (int k = 0; k < q_n_frames; ++k) {
      // row blocks whose last token lies in chunk frame k
      const int64_t end = k + 1 < q_n_frames ? ((k + 1) * T) / rpb : f.n_rb;
      const int64_t start = c.n == 0 ? 0 : c.rb_end[c.n - 1];
      if (end <= start) continue;
      const int64_t frames = (int64_t)s->window_frames - (q_n_frames - 1 - k);
      const int nt = (int)(frames < 1 ? 1 : (frames * T + tk - 1) / tk);
      c.rb_end[c.n] = (int)end;
      c.nt[c.n] = nt;
      c.u0[c.n] = u;
      u += (end - start) * nt;
      ++c.n;
    }
    c.per_stream = u;
  } else {
    c.n = 1;
    c.rb_end[0] = f.n_rb;
    c.nt[0] = f.nt_max;
    c.u0[0] = 0;
    c.per_stream = (int64_t)f.n_rb * f.nt_max;
  }
  const int64_t pairs = (int64_t)s->batch * s->n_heads;
  const int64_t row_blocks = pairs * f.n_rb;
  f.units = pairs * c.per_stream;
  int64_t g = device_cus();
  if (g > f.units) g = f.units;
  if (g > (mla::kMaxMergePieces - 1) * row_blocks) g = (mla::kMaxMergePieces - 1) * row_blocks;
  if (g < 1) g = 1;
  f.grid = (int)g;
  // whole row blocks in rounds where there are enough of them, the rest shared
  f.rb_whole = row_blocks >= g ? row_blocks / g * g : 0;
  long long u_rest;
  int nt_unused;
  mla::row_block_units(c, f.n_rb, f.rb_whole, u_rest, nt_unused);  // (rb_whole = all row blocks: U)
  f.u_rest = u_rest;
  const int64_t rest = f.units - f.u_rest;
  int64_t gr = g;
  if (f.rb_whole > 0) {
    const int64_t rb_rest = row_blocks - f.rb_whole;
    if (gr > (mla::kMaxMergePieces - 1) * rb_rest) gr = (mla::kMaxMergePieces - 1) * rb_rest;
    if (gr > rest) gr = rest;
  }
  f.grid_rest = (int)gr;
  f.split = c.n > 1 || (rest > 0 && !(rest % gr == 0 && (rest / gr) % f.nt_max == 0));
  return f;
}

// Per-head form workspace: fallback count and row list, the window's rotated
// kR, the expanded keys and values of every head, the concatenated queries,
// and the partial-result slots of split row blocks.
struct HeadsWs {
  size_t count, rows, krot, k_exp, v_exp, q_cat, part_o, part_l, total;
};

HeadsWs heads_ws_layout(const mla_shape* s, int q_n_frames) {
  const size_t nq = (size_t)q_n_frames * tokens_per_frame(s);
  const size_t nk = (size_t)s->window_frames * tokens_per_frame(s);
  const size_t e = elt_size(s);
  HeadsWs w;
  w.count = 0;
  w.rows = 256;
  w.krot = w.rows + round256((size_t)s->batch * s->n_heads * nq * sizeof(int));
  w.k_exp = w.krot + round256((size_t)s->batch * nk * s->d_rope * e);
  w.v_exp = w.k_exp + round256((size_t)s->batch * s->n_heads * nk * s->d_head * e);
  w.q_cat = w.v_exp + round256((size_t)s->batch * s->n_heads * nk * s->d_head * e);
  w.part_o = w.q_cat + round256((size_t)s->batch * s->n_heads * nq * (s->d_head + s->d_rope) * e);
  // partial slots for either mask (the frame-causal plan may split row
  // blocks where the plain one does not)
  size_t slots = 0;
  for (const bool causal : {false, true}) {
    const FlashPlan f = heads_plan(s, q_n_frames, causal);
    const size_t n = f.split ? (size_t)f.grid * 2 * mla::kHeadsRowsPerBlock : 0;
    slots = n > slots ? n : slots;
  }
  w.part_l = w.part_o + round256(slots * s->d_head * e);
  w.total = w.part_l + round256(slots * 2 * sizeof(float));
  return w;
}

}  // namespace

MLA_API int32_t mla_abi_version(void) { return MLA_ABI_VERSION; }

MLA_API const char* mla_status_string(int32_t status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_NULL: return "a required pointer is NULL";
    case MLA_ERR_SHAPE: return "dimensions inconsistent or out of range";
    case MLA_ERR_DTYPE: return "dtype must be MLA_BF16 or MLA_F32";
    case MLA_ERR_ALIGN: return "a device pointer is not 16-byte aligned";
    case MLA_ERR_WORKSPACE: return "workspace too small";
    case MLA_ERR_UNSUPPORTED: return "(d_c, d_rope) has no kernel instantiation";
    case MLA_ERR_HIP: return "HIP launch failed";
    case MLA_ERR_RANGE: return "frame or table index out of range";
    case MLA_ERR_SCRATCH: return "the call needs more scratch than the library's fixed per-device buffer holds";
    default: return "unknown status";
  }
}

MLA_API mla_status mla_shape_check(const mla_shape* shape) { return check_shape(shape); }

MLA_API int32_t mla_qabs_dim(const mla_shape* shape) {
  return check_shape(shape) == MLA_OK ? qabs_dim(shape) : 0;
}

MLA_API size_t mla_rope3d_table_floats(const mla_shape* shape, int32_t n_t) {
  if (check_shape(shape) != MLA_OK || n_t < 1) return 0;
  return table_floats(shape, n_t);
}

MLA_API mla_status mla_rope3d_tables(const mla_shape* shape, int32_t t_first, int32_t n_t, float* tables,
                                     void* stream) {
  mla_status st = check_shape(shape);
  if (st != MLA_OK) return st;
  if (!tables) return MLA_ERR_NULL;
  if (!aligned16(tables)) return MLA_ERR_ALIGN;
  if (n_t < 1 || t_first < 0 || (int64_t)t_first + n_t > INT32_MAX) return MLA_ERR_RANGE;
  mla::RopeTableParams p;
  p.tables = tables;
  p.rl = rope_layout(shape, t_first, n_t);
  p.grid_y = shape->grid_y;
  p.grid_x = shape->grid_x;
  p.base = (double)shape->rope_base;
  p.total = (int)(table_floats(shape, n_t) / 2);
  return from_hip(mla::launch_rope_tables(p, (hipStream_t)stream));
}

// Each *_impl validates, then (run = true) enqueues; with run = false it
// only validates, so that a composite call can check every part before it
// enqueues anything.
static mla_status cache_write_impl(const mla_shape* shape, const void* x, const void* w_dkv, const void* w_kr,
                                   int32_t frame_first, int32_t n_frames, void* cache, int32_t* slot_frame,
                                   void* stream, bool run) {
  mla_status st = check_shape(shape);
  if (st != MLA_OK) return st;
  if (!x || !w_dkv || !w_kr || !cache || !slot_frame) return MLA_ERR_NULL;
  if (!aligned16(x) || !aligned16(w_dkv) || !aligned16(w_kr) || !aligned16(cache) || !aligned16(slot_frame))
    return MLA_ERR_ALIGN;
  if (frame_first < 0 || n_frames < 1 || n_frames > shape->window_frames ||
      (int64_t)frame_first + n_frames > INT32_MAX)
    return MLA_ERR_RANGE;
  const int64_t rows = (int64_t)shape->batch * n_frames * tokens_per_frame(shape);
  if (rows > INT32_MAX / 2) return MLA_ERR_SHAPE;
  if (!run) return MLA_OK;
  mla::CacheWriteParams p;
  p.x = x;
  p.w_dkv = w_dkv;
  p.w_kr = w_kr;
  p.cache = cache;
  p.slot_frame = slot_frame;
  p.rows = (int)rows;
  p.rows_per_b = (int)(n_frames * tokens_per_frame(shape));
  p.hidden = shape->hidden;
  p.d_c = shape->d_c;
  p.d_rope = shape->d_rope;
  p.W = shape->window_frames;
  p.T = (int)tokens_per_frame(shape);
  p.frame_first = frame_first;
  p.n_frames = n_frames;
  p.batch = shape->batch;
  return from_hip(mla::launch_cache_write(shape->dtype, shape->d_c, shape->d_rope, p, (hipStream_t)stream));
}

MLA_API mla_status mla_cache_write(const mla_shape* shape, const void* x, const void* w_dkv, const void* w_kr,
                                   int32_t frame_first, int32_t n_frames, void* cache, int32_t* slot_frame,
                                   void* stream) {
  return cache_write_impl(shape, x, w_dkv, w_kr, frame_first, n_frames, cache, slot_frame, stream, true);
}

MLA_API mla_status mla_absorb_q(const mla_shape* shape, const void* q_nope, const void* q_r, int32_t q_frame_first,
                                int32_t q_n_frames, const void* w_uk, const float* rope_tables,
                                int32_t rope_t_first, int32_t rope_n_t, void* q_abs, void* stream) {
  mla_status st = check_shape(shape);
  if (st != MLA_OK) return st;
  if (!q_nope || !q_r || !w_uk || !q_abs) return MLA_ERR_NULL;
  if (!aligned16(q_nope) || !aligned16(q_r) || !aligned16(w_uk) || !aligned16(q_abs)) return MLA_ERR_ALIGN;
  if ((st = check_tables(shape, rope_tables, rope_t_first, rope_n_t)) != MLA_OK) return st;
  if ((st = check_query_args(shape, q_frame_first, q_n_frames)) != MLA_OK) return st;
  if (q_frame_first < rope_t_first || (int64_t)q_frame_first + q_n_frames > (int64_t)rope_t_first + rope_n_t)
    return MLA_ERR_RANGE;
  return do_absorb(shape, q_nope, q_r, q_frame_first, q_n_frames, w_uk, rope_tables, rope_t_first, rope_n_t, q_abs,
                   (hipStream_t)stream);
}

MLA_API size_t mla_flash_workspace_bytes(const mla_shape* shape, int32_t q_n_frames, int32_t kv_splits) {
  // 0 for any shape or chunk size that the calls themselves reject
  if (check_shape(shape) != MLA_OK || check_query_args(shape, 0, q_n_frames) != MLA_OK || kv_splits < 0 ||
      kv_splits > kMaxSplits)
    return 0;
  return flash_ws_bytes(shape, q_n_frames, kv_splits);
}

static mla_status flash_attend_impl(const mla_shape* shape, const void* q_abs, int32_t q_frame_first,
                                    int32_t q_n_frames, const void* cache, const int32_t* slot_frame,
                                    const float* rope_tables, int32_t rope_t_first, int32_t rope_n_t, void* o_lat,
                                    int32_t kv_splits, void* workspace, size_t workspace_bytes, void* stream,
                                    bool frame_causal) {
  mla_status st = check_shape(shape);
  if (st != MLA_OK) return st;
  if (!q_abs || !cache || !slot_frame || !o_lat) return MLA_ERR_NULL;
  if (!aligned16(q_abs) || !aligned16(cache) || !aligned16(slot_frame) || !aligned16(o_lat)) return MLA_ERR_ALIGN;
  if ((st = check_tables(shape, rope_tables, rope_t_first, rope_n_t)) != MLA_OK) return st;
  if ((st = check_query_args(shape, q_frame_first, q_n_frames)) != MLA_OK) return st;
  if (kv_splits < 0 || kv_splits > kMaxSplits) return MLA_ERR_RANGE;
  if (!workspace) return MLA_ERR_NULL;
  if (!aligned16(workspace)) return MLA_ERR_ALIGN;
  if (!flash_plan_ok(flash_plan(shape, q_n_frames, kv_splits))) return MLA_ERR_SHAPE;
  if (workspace_bytes < flash_ws_bytes(shape, q_n_frames, kv_splits)) return MLA_ERR_WORKSPACE;
  return do_flash(shape, q_abs, q_n_frames, cache, slot_frame, rope_tables, rope_t_first, rope_n_t, o_lat, kv_splits,
                  workspace, (hipStream_t)stream, frame_causal, q_frame_first);
}

MLA_API mla_status mla_flash_attend(const mla_shape* shape, const void* q_abs, int32_t q_n_frames, const void* cache,
                                    const int32_t* slot_frame, const float* rope_tables, int32_t rope_t_first,
                                    int32_t rope_n_t, void* o_lat, int32_t kv_splits, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  return flash_attend_impl(shape, q_abs, 0, q_n_frames, cache, slot_frame, rope_tables, rope_t_first, rope_n_t, o_lat,
                           kv_splits, workspace, workspace_bytes, stream, false);
}

MLA_API mla_status mla_flash_attend_frame_causal(const mla_shape* shape, const void* q_abs, int32_t q_frame_first,
                                                 int32_t q_n_frames, const void* cache, const int32_t* slot_frame,
                                                 const float* rope_tables, int32_t rope_t_first, int32_t rope_n_t,
                                                 void* o_lat, int32_t kv_splits, void* workspace,
                                                 size_t workspace_bytes, void* stream) {
  return flash_attend_impl(shape, q_abs, q_frame_first, q_n_frames, cache, slot_frame, rope_tables, rope_t_first,
                           rope_n_t, o_lat, kv_splits, workspace, workspace_bytes, stream, true);
}

// Argument checks and launch of mla_flash_attend with the workspace supplied
// separately (the allocation-free entry point keeps its own).
mla_status mla_abi::flash_check(const mla_shape* shape, const void* q_abs, int32_t q_n_frames, const void* cache,
                                const int32_t* slot_frame, const float* rope_tables, int32_t rope_t_first,
                                int32_t rope_n_t, const void* o_lat, int32_t kv_splits, size_t* ws_bytes) {
  mla_status st = check_shape(shape);
  if (st != MLA_OK) return st;
  if (!q_abs || !cache || !slot_frame || !o_lat) return MLA_ERR_NULL;
  if (!aligned16(q_abs) || !aligned16(cache) || !aligned16(slot_frame) || !aligned16(o_lat)) return MLA_ERR_ALIGN;
  if ((st = check_tables(shape, rope_tables, rope_t_first, rope_n_t)) != MLA_OK) return st;
  if ((st = check_query_args(shape, 0, q_n_frames)) != MLA_OK) return st;
  if (kv_splits < 0 || kv_splits > kMaxSplits) return MLA_ERR_RANGE;
  if (!flash_plan_ok(flash_plan(shape, q_n_frames, kv_splits))) return MLA_ERR_SHAPE;
  *ws_bytes = flash_ws_bytes(shape, q_n_frames, kv_splits);
  return MLA_OK;
}

mla_status mla_abi::flash_run(const mla_shape* shape, const void* q_abs, int32_t q_n_frames, const void* cache,
                              const int32_t* slot_frame, const float* rope_tables, int32_t rope_t_first,
                              int32_t rope_n_t, void* o_lat, int32_t kv_splits, void* workspace, void* stream) {
  return do_flash(shape, q_abs, q_n_frames, cache, slot_frame, rope_tables, rope_t_first, rope_n_t, o_lat, kv_splits,
                  workspace, (hipStream_t)stream);
}

MLA_API mla_status mla_up_v(const mla_shape* shape, const void* o_lat, int32_t q_n_frames, const void* w_uv,
                            void* out, void* stream) {
  mla_status st = check_shape(shape);
  if (st != MLA_OK) return st;
  if (!o_lat || !w_uv || !out) return MLA_ERR_NULL;
  if (!aligned16(o_lat) || !aligned16(w_uv) || !aligned16(out)) return MLA_ERR_ALIGN;
  if ((st = check_query_args(shape, 0, q_n_frames)) != MLA_OK) return st;
  return do_up_v(shape, o_lat, q_n_frames, w_uv, out, (hipStream_t)stream);
}

// Workspace of the latent form: [q_abs | o_lat | flash workspace].
static size_t latent_ws_bytes(const mla_shape* shape, int32_t q_n_frames) {
  const size_t rows = (size_t)shape->batch * q_n_frames * tokens_per_frame(shape) * shape->n_heads;
  return round256(rows * qabs_dim(shape) * elt_size(shape)) + round256(rows * shape->d_c * elt_size(shape)) +
         flash_ws_bytes(shape, q_n_frames, 0);
}

static size_t heads_ws_bytes(const mla_shape* shape, int32_t q_n_frames);

// The form mla_chunk_attend takes. The per-head form does
// 2 d_head + d_rope products per (query, key, head) against the latent
// form's 2 d_c + d_rope, plus a per-call expansion of the window's keys and
// values (4 d_head d_c products per key and head) that only a large enough
// chunk repays: it is taken where it is supported, saves at least 20% of the
// products, and the chunk has at least 2048 query tokens per stream.
// Measured with both forms' kernels as they are (latent form in the step,
// clock settled): at the Wan2.1 width (d_c 192, d_rope 32) the per-head form
// is 1.15x faster at a 3-frame chunk (4680 queries), 1.07x at 2 frames
// (3120) and 0.96x at 1 frame (1560); 1.14x at (192, 64), 1.00x at
// (160, 64) (products ratio 1.2) and 0.76x at (128, 32) (ratio 1.0).
constexpr double kHeadsMinProductRatio = 1.25;
constexpr int64_t kHeadsMinQueries = 2048;

static bool heads_preferred(const mla_shape* s, int32_t q_n_frames) {
  if (!mla::heads_supported(s->dtype == MLA_BF16 ? 0 : 1, s->d_c, s->d_rope, s->d_head)) return false;
  const double ratio = (2.0 * s->d_c + s->d_rope) / (2.0 * s->d_head + s->d_rope);
  return ratio >= kHeadsMinProductRatio && (int64_t)q_n_frames * tokens_per_frame(s) >= kHeadsMinQueries;
}

MLA_API int32_t mla_chunk_attend_form(const mla_shape* shape, int32_t q_n_frames) {
  if (check_shape(shape) != MLA_OK || check_query_args(shape, 0, q_n_frames) != MLA_OK) return -1;
  return heads_preferred(shape, q_n_frames) ? MLA_FORM_HEADS : MLA_FORM_LATENT;
}

MLA_API size_t mla_chunk_attend_workspace_bytes(const mla_shape* shape, int32_t q_n_frames) {
  if (check_shape(shape) != MLA_OK || check_query_args(shape, 0, q_n_frames) != MLA_OK) return 0;
  size_t n = latent_ws_bytes(shape, q_n_frames);
  if (heads_preferred(shape, q_n_frames)) {
    const size_t h = heads_ws_bytes(shape, q_n_frames);
    n = h > n ? h : n;
  }
  return n;
}

// Attention over the window from absorbed queries (mla_flash_attend with the
// automatic split, then mla_up_v); workspace = [o_lat | flash workspace].
static size_t attend_absorbed_ws_bytes(const mla_shape* shape, int32_t q_n_frames) {
  const size_t rows = (size_t)shape->batch * q_n_frames * tokens_per_frame(shape) * shape->n_heads;
  return round256(rows * shape->d_c * elt_size(shape)) + flash_ws_bytes(shape, q_n_frames, 0);
}

static mla_status attend_absorbed_impl(const mla_shape* shape, const void* q_abs, int32_t q_frame_first,
                                       int32_t q_n_frames, const void* w_uv, const void* cache,
                                       const int32_t* slot_frame, const float* rope_tables, int32_t rope_t_first,
                                       int32_t rope_n_t, void* out, void* workspace, size_t workspace_bytes,
                                       void* stream, bool frame_causal, bool run) {
  mla_status st = check_shape(shape);
  if (st != MLA_OK) return st;
  if (!q_abs || !w_uv || !cache || !slot_frame || !out || !workspace) return MLA_ERR_NULL;
  if (!aligned16(q_abs) || !aligned16(w_uv) || !aligned16(cache) || !aligned16(slot_frame) || !aligned16(out) ||
      !aligned16(workspace))
    return MLA_ERR_ALIGN;
  if ((st = check_tables(shape, rope_tables, rope_t_first, rope_n_t)) != MLA_OK) return st;
  if ((st = check_query_args(shape, q_frame_first, q_n_frames)) != MLA_OK) return st;
  if (q_frame_first < rope_t_first || (int64_t)q_frame_first + q_n_frames > (int64_t)rope_t_first + rope_n_t)
    return MLA_ERR_RANGE;
  if (!flash_plan_ok(flash_plan(shape, q_n_frames, 0))) return MLA_ERR_SHAPE;
  if (workspace_bytes < attend_absorbed_ws_bytes(shape, q_n_frames)) return MLA_ERR_WORKSPACE;
  if (!run) return MLA_OK;
  const size_t rows = (size_t)shape->batch * q_n_frames * tokens_per_frame(shape) * shape->n_heads;
  char* ws = (char*)workspace;
  void* o_lat = ws;
  ws += round256(rows * shape->d_c * elt_size(shape));
  hipStream_t s = (hipStream_t)stream;
  if ((st = do_flash(shape, q_abs, q_n_frames, cache, slot_frame, rope_tables, rope_t_first, rope_n_t, o_lat, 0,
                     ws, s, frame_causal, q_frame_first)) != MLA_OK)
    return st;
  return do_up_v(shape, o_lat, q_n_frames, w_uv, out, s);
}

static mla_status chunk_attend_impl(const mla_shape* shape, const void* q_nope, const void* q_r,
                                    int32_t q_frame_first, int32_t q_n_frames, const void* w_uk, const void* w_uv,
                                    const void* cache, const int32_t* slot_frame, const float* rope_tables,
                                    int32_t rope_t_first, int32_t rope_n_t, void* out, void* workspace,
                                    size_t workspace_bytes, void* stream, bool frame_causal, bool run = true) {
  mla_status st = check_shape(shape);
  if (st != MLA_OK) return st;
  if (!q_nope || !q_r || !w_uk || !w_uv || !cache || !slot_frame || !out || !workspace) return MLA_ERR_NULL;
  if (!aligned16(q_nope) || !aligned16(q_r) || !aligned16(w_uk) || !aligned16(w_uv) || !aligned16(cache) ||
      !aligned16(slot_frame) || !aligned16(out) || !aligned16(workspace))
    return MLA_ERR_ALIGN;
  if ((st = check_tables(shape, rope_tables, rope_t_first, rope_n_t)) != MLA_OK) return st;
  if ((st = check_query_args(shape, q_frame_first, q_n_frames)) != MLA_OK) return st;
  if (q_frame_first < rope_t_first || (int64_t)q_frame_first + q_n_frames > (int64_t)rope_t_first + rope_n_t)
    return MLA_ERR_RANGE;
  if (!flash_plan_ok(flash_plan(shape, q_n_frames, 0))) return MLA_ERR_SHAPE;
  if (workspace_bytes < latent_ws_bytes(shape, q_n_frames)) return MLA_ERR_WORKSPACE;
  // workspace = [q_abs | o_lat | flash workspace]
  const size_t rows = (size_t)shape->batch * q_n_frames * tokens_per_frame(shape) * shape->n_heads;
  const size_t qabs_bytes = round256(rows * qabs_dim(shape) * elt_size(shape));
  char* ws = (char*)workspace;
  if ((st = attend_absorbed_impl(shape, ws, q_frame_first, q_n_frames, w_uv, cache, slot_frame, rope_tables,
                                 rope_t_first, rope_n_t, out, ws + qabs_bytes, workspace_bytes - qabs_bytes, stream,
                                 frame_causal, false)) != MLA_OK)
    return st;
  if (!run) return MLA_OK;
  if ((st = do_absorb(shape, q_nope, q_r, q_frame_first, q_n_frames, w_uk, rope_tables, rope_t_first, rope_n_t, ws,
                      (hipStream_t)stream)) != MLA_OK)
    return st;
  return attend_absorbed_impl(shape, ws, q_frame_first, q_n_frames, w_uv, cache, slot_frame, rope_tables,
                              rope_t_first, rope_n_t, out, ws + qabs_bytes, workspace_bytes - qabs_bytes, stream,
                              frame_causal, true);
}

static mla_status chunk_attend_heads_impl(const mla_shape* shape, const void* q_nope, const void* q_r,
                                          int32_t q_frame_first, int32_t q_n_frames, const void* w_uk,
                                          const void* w_uv, const void* cache, const int32_t* slot_frame,
                                          const float* rope_tables, int32_t rope_t_first, int32_t rope_n_t, void* out,
                                          void* workspace, size_t workspace_bytes, void* stream, bool run,
                                          bool frame_causal);

MLA_API mla_status mla_chunk_attend(const mla_shape* shape, const void* q_nope, const void* q_r, int32_t q_frame_first,
                                    int32_t q_n_frames, const void* w_uk, const void* w_uv, const void* cache,
                                    const int32_t* slot_frame, const float* rope_tables, int32_t rope_t_first,
                                    int32_t rope_n_t, void* out, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  mla_status st = check_shape(shape);
  if (st != MLA_OK) return st;
  if ((st = check_query_args(shape, q_frame_first, q_n_frames)) != MLA_OK) return st;
  if (heads_preferred(shape, q_n_frames))
    return chunk_attend_heads_impl(shape, q_nope, q_r, q_frame_first, q_n_frames, w_uk, w_uv, cache, slot_frame,
                                   rope_tables, rope_t_first, rope_n_t, out, workspace, workspace_bytes, stream, true,
                                   false);
  return chunk_attend_impl(shape, q_nope, q_r, q_frame_first, q_n_frames, w_uk, w_uv, cache, slot_frame, rope_tables,
                           rope_t_first, rope_n_t, out, workspace, workspace_bytes, stream, false);
}

MLA_API mla_status mla_chunk_attend_latent(const mla_shape* shape, const void* q_nope, const void* q_r,
                                           int32_t q_frame_first, int32_t q_n_frames, const void* w_uk,
                                           const void* w_uv, const void* cache, const int32_t* slot_frame,
                                           const float* rope_tables, int32_t rope_t_first, int32_t rope_n_t,
                                           void* out, void* workspace, size_t workspace_bytes, void* stream) {
  return chunk_attend_impl(shape, q_nope, q_r, q_frame_first, q_n_frames, w_uk, w_uv, cache, slot_frame, rope_tables,
                           rope_t_first, rope_n_t, out, workspace, workspace_bytes, stream, false);
}

MLA_API mla_status mla_chunk_attend_frame_causal(const mla_shape* shape, const void* q_nope, const void* q_r,
                                                 int32_t q_frame_first, int32_t q_n_frames, const void* w_uk,
                                                 const void* w_uv, const void* cache, const int32_t* slot_frame,
                                                 const float* rope_tables, int32_t rope_t_first, int32_t rope_n_t,
                                                 void* out, void* workspace, size_t workspace_bytes, void* stream) {
  mla_status st = check_shape(shape);
  if (st != MLA_OK) return st;
  if ((st = check_query_args(shape, q_frame_first, q_n_frames)) != MLA_OK) return st;
  if (heads_preferred(shape, q_n_frames))
    return chunk_attend_heads_impl(shape, q_nope, q_r, q_frame_first, q_n_frames, w_uk, w_uv, cache, slot_frame,
                                   rope_tables, rope_t_first, rope_n_t, out, workspace, workspace_bytes, stream, true,
                                   true);
  return chunk_attend_impl(shape, q_nope, q_r, q_frame_first, q_n_frames, w_uk, w_uv, cache, slot_frame, rope_tables,
                           rope_t_first, rope_n_t, out, workspace, workspace_bytes, stream, true);
}

MLA_API mla_status mla_chunk_attend_latent_frame_causal(const mla_shape* shape, const void* q_nope, const void* q_r,
                                                        int32_t q_frame_first, int32_t q_n_frames, const void* w_uk,
                                                        const void* w_uv, const void* cache,
                                                        const int32_t* slot_frame, const float* rope_tables,
                                                        int32_t rope_t_first, int32_t rope_n_t, void* out,
                                                        void* workspace, size_t workspace_bytes, void* stream) {
  return chunk_attend_impl(shape, q_nope, q_r, q_frame_first, q_n_frames, w_uk, w_uv, cache, slot_frame, rope_tables,
                           rope_t_first, rope_n_t, out, workspace, workspace_bytes, stream, true);
}

static size_t heads_ws_bytes(const mla_shape* shape, int32_t q_n_frames) {
  return heads_ws_layout(shape, q_n_frames).total;
}

MLA_API size_t mla_chunk_attend_heads_workspace_bytes(const mla_shape* shape, int32_t q_n_frames) {
  if (check_shape(shape) != MLA_OK || check_query_args(shape, 0, q_n_frames) != MLA_OK) return 0;
  if (!mla::heads_supported(shape->dtype == MLA_BF16 ? 0 : 1, shape->d_c, shape->d_rope, shape->d_head)) return 0;
  return heads_ws_bytes(shape, q_n_frames);
}

MLA_API mla_status mla_chunk_attend_heads(const mla_shape* shape, const void* q_nope, const void* q_r,
                                          int32_t q_frame_first, int32_t q_n_frames, const void* w_uk,
                                          const void* w_uv, const void* cache, const int32_t* slot_frame,
                                          const float* rope_tables, int32_t rope_t_first, int32_t rope_n_t,
                                          void* out, void* workspace, size_t workspace_bytes, void* stream) {
  return chunk_attend_heads_impl(shape, q_nope, q_r, q_frame_first, q_n_frames, w_uk, w_uv, cache, slot_frame,
                                 rope_tables, rope_t_first, rope_n_t, out, workspace, workspace_bytes, stream, true,
                                 false);
}

MLA_API mla_status mla_chunk_attend_heads_frame_causal(const mla_shape* shape, const void* q_nope, const void* q_r,
                                                       int32_t q_frame_first, int32_t q_n_frames, const void* w_uk,
                                                       const void* w_uv, const void* cache, const int32_t* slot_frame,
                                                       const float* rope_tables, int32_t rope_t_first,
                                                       int32_t rope_n_t, void* out, void* workspace,
                                                       size_t workspace_bytes, void* stream) {
  return chunk_attend_heads_impl(shape, q_nope, q_r, q_frame_first, q_n_frames, w_uk, w_uv, cache, slot_frame,
                                 rope_tables, rope_t_first, rope_n_t, out, workspace, workspace_bytes, stream, true,
                                 true);
}

static mla_status chunk_attend_heads_impl(const mla_shape* shape, const void* q_nope, const void* q_r,
                                          int32_t q_frame_first, int32_t q_n_frames, const void* w_uk,
                                          const void* w_uv, const void* cache, const int32_t* slot_frame,
                                          const float* rope_tables, int32_t rope_t_first, int32_t rope_n_t, void* out,
                                          void* workspace, size_t workspace_bytes, void* stream, bool run,
                                          bool frame_causal) {
  mla_status st = check_shape(shape);
  if (st != MLA_OK) return st;
  if (!mla::heads_supported(shape->dtype == MLA_BF16 ? 0 : 1, shape->d_c, shape->d_rope, shape->d_head))
    return MLA_ERR_UNSUPPORTED;
  if (!q_nope || !q_r || !w_uk || !w_uv || !cache || !slot_frame || !out || !workspace) return MLA_ERR_NULL;
  if (!aligned16(q_nope) || !aligned16(q_r) || !aligned16(w_uk) || !aligned16(w_uv) || !aligned16(cache) ||
      !aligned16(slot_frame) || !aligned16(out) || !aligned16(workspace))
    return MLA_ERR_ALIGN;
  if ((st = check_tables(shape, rope_tables, rope_t_first, rope_n_t)) != MLA_OK) return st;
  if ((st = check_query_args(shape, q_frame_first, q_n_frames)) != MLA_OK) return st;
  if (q_frame_first < rope_t_first || (int64_t)q_frame_first + q_n_frames > (int64_t)rope_t_first + rope_n_t)
    return MLA_ERR_RANGE;
  const FlashPlan f = heads_plan(shape, q_n_frames, frame_causal);
  if (!flash_plan_ok(f)) return MLA_ERR_SHAPE;
  const HeadsWs w = heads_ws_layout(shape, q_n_frames);
  if (workspace_bytes < w.total) return MLA_ERR_WORKSPACE;
  if (!run) return MLA_OK;
  char* base = (char*)workspace;
  hipStream_t s = (hipStream_t)stream;
  const int T = (int)tokens_per_frame(shape);
  // rotated kR of the window (and the fallback count cleared) by the latent
  // form's rotation pass
  mla::FlashParams fp = {};
  fp.cache = cache;
  fp.slot_frame = slot_frame;
  fp.tables = rope_tables;
  fp.krot = base + w.krot;
  fp.fallback_count = (int*)(base + w.count);
  fp.rl = rope_layout(shape, rope_t_first, rope_n_t);
  fp.W = shape->window_frames;
  fp.T = T;
  fp.grid_y = shape->grid_y;
  fp.grid_x = shape->grid_x;
  fp.batch = shape->batch;
  fp.rope_base = (double)shape->rope_base;
  hipError_t e = mla::launch_rope_window(shape->dtype == MLA_BF16 ? 0 : 1, shape->d_c, shape->d_rope, fp, s);
  if (e != hipSuccess) return MLA_ERR_HIP;
  mla::HeadsParams p = {};
  p.q_nope = q_nope;
  p.q_r = q_r;
  p.w_uk = w_uk;
  p.w_uv = w_uv;
  p.cache = cache;
  p.slot_frame = slot_frame;
  p.tables = rope_tables;
  p.out = out;
  p.q_cat = base + w.q_cat;
  p.k_exp = base + w.k_exp;
  p.v_exp = base + w.v_exp;
  p.krot = base + w.krot;
  p.fallback_count = (int*)(base + w.count);
  p.fallback_rows = (int*)(base + w.rows);
  p.rl = fp.rl;
  p.batch = shape->batch;
  p.H = shape->n_heads;
  p.Nq = (int)(q_n_frames * T);
  p.T = T;
  p.W = shape->window_frames;
  p.grid_x = shape->grid_x;
  p.q_frame_first = q_frame_first;
  p.part_o = f.split ? (void*)(base + w.part_o) : nullptr;
  p.part_l = f.split ? (float*)(base + w.part_l) : nullptr;
  p.n_rb = f.n_rb;
  p.nt_max = f.nt_max;
  p.units = f.units;
  p.classes = f.classes;
  p.grid = f.grid;
  p.rb_whole = f.rb_whole;
  p.u_rest = f.u_rest;
  p.grid_rest = f.grid_rest;
  p.qscale = scale_log2(shape);
  return from_hip(mla::launch_heads(shape->d_c, shape->d_rope, shape->d_head, p, f.split, frame_causal, s));
}


namespace {

constexpr int kMaxQueryLatent = 1 << 16;

// work-group tiles of a projection (at most 64 x 64 outputs each) are counted in 32 bits
mla_status check_gemm_tiles(int64_t M, int64_t N) {
  return ((M + 63) / 64) * ((N + 63) / 64) > (INT64_C(1) << 30) ? MLA_ERR_SHAPE : MLA_OK;
}

// C = A B^T with the output features split in two parts (n >= n_split: weight
// b2, output c2); n_split = N for a single part.
mla_status gemm(const mla_shape* s, const void* a, const void* b, const void* b2, void* c, void* c2, int64_t M,
                int N, int n_split, int K, hipStream_t st) {
  if (check_gemm_tiles(M, N) != MLA_OK) return MLA_ERR_SHAPE;
  mla::GemmParams p{};
  p.a = a;
  p.b = b;
  p.b2 = b2;
  p.c = c;
  p.c2 = c2;
  p.M = (int)M;
  p.N = N;
  p.K = K;
  p.lda = K;
  p.ldb = K;
  p.ldc = n_split;
  p.ldc2 = N - n_split;
  p.n_split = n_split;
  p.n_split2 = N;
  return from_hip(mla::launch_gemm_nt(s->dtype, p, mla::gemm_tile_rows(p.M, N, device_cus()), st));
}

// The query latent and the cache write of the same tokens in one product:
// x [W_dq ; W_dkv ; W_kR]^T, the first d_cq features into c_q, the rest
// ([c | kR] of each token) into ring slot f mod W of its frame f, which the
// kernel also records in slot_frame. Arguments checked by the callers.
mla_status gemm_query_latent_and_cache(const mla_shape* s, int d_cq, const void* x, const void* w_dq,
                                       const void* w_dkv, const void* w_kr, int frame_first, int n_frames,
                                       void* c_q, void* cache, int32_t* slot_frame, hipStream_t st) {
  const int64_t M = (int64_t)s->batch * n_frames * tokens_per_frame(s);
  const int N = d_cq + s->d_c + s->d_rope;
  if (check_gemm_tiles(M, N) != MLA_OK) return MLA_ERR_SHAPE;
  mla::GemmParams p{};
  p.a = x;
  p.b = w_dq;
  p.b2 = w_dkv;
  p.b3 = w_kr;
  p.c = c_q;
  p.c2 = cache;
  p.M = (int)M;
  p.N = N;
  p.K = s->hidden;
  p.lda = s->hidden;
  p.ldb = s->hidden;
  p.ldc = d_cq;
  p.ldc2 = s->d_c + s->d_rope;
  p.n_split = d_cq;
  p.n_split2 = d_cq + s->d_c;
  p.ring.slot_frame = slot_frame;
  p.ring.rows_per_b = (int)(n_frames * tokens_per_frame(s));
  p.ring.T = (int)tokens_per_frame(s);
  p.ring.W = s->window_frames;
  p.ring.frame_first = frame_first;
  p.ring.n_frames = n_frames;
  p.ring.batch = s->batch;
  return from_hip(mla::launch_gemm_ring(s->dtype, p, mla::gemm_tile_rows(p.M, N, device_cus()), st));
}

mla_status check_projection_rows(const mla_shape* s, int n_frames, int64_t* rows) {
  if (n_frames < 1) return MLA_ERR_RANGE;
  *rows = (int64_t)s->batch * n_frames * tokens_per_frame(s);
  if (*rows > INT32_MAX / 2) return MLA_ERR_SHAPE;
  return MLA_OK;
}

}  // namespace

// cq_ready: c_q already holds the query latent (the layer step computes it
// together with the cache write); only the per-head queries are launched.
static mla_status query_project_impl(const mla_shape* shape, int32_t d_cq, const void* x, int32_t n_frames,
                                     const void* w_dq, const void* w_uq, const void* w_qr, void* c_q, void* q_nope,
                                     void* q_r, void* stream, bool run, bool cq_ready = false) {
  mla_status st = check_shape(shape);
  if (st != MLA_OK) return st;
  if (!x || !w_dq || !w_uq || !w_qr || !c_q || !q_nope || !q_r) return MLA_ERR_NULL;
  if (!aligned16(x) || !aligned16(w_dq) || !aligned16(w_uq) || !aligned16(w_qr) || !aligned16(c_q) ||
      !aligned16(q_nope) || !aligned16(q_r))
    return MLA_ERR_ALIGN;
  if (d_cq < 8 || d_cq % 8 != 0 || d_cq > kMaxQueryLatent) return MLA_ERR_SHAPE;
  if ((int64_t)shape->n_heads * (shape->d_head + shape->d_rope) > kMaxQueryLatent || shape->d_rope % 8 != 0)
    return MLA_ERR_SHAPE;
  int64_t rows = 0;
  if ((st = check_projection_rows(shape, n_frames, &rows)) != MLA_OK) return st;
  const int n_nope = shape->n_heads * shape->d_head;
  if ((st = check_gemm_tiles(rows, d_cq)) != MLA_OK ||
      (st = check_gemm_tiles(rows, n_nope + shape->n_heads * shape->d_rope)) != MLA_OK)
    return st;
  if (!run) return MLA_OK;
  hipStream_t s = (hipStream_t)stream;
  if (!cq_ready && (st = gemm(shape, x, w_dq, nullptr, c_q, nullptr, rows, d_cq, d_cq, shape->hidden, s)) != MLA_OK)
    return st;
  // content and positional queries in one product over the same query latent
  return gemm(shape, c_q, w_uq, w_qr, q_nope, q_r, rows, n_nope + shape->n_heads * shape->d_rope, n_nope, d_cq, s);
}

MLA_API mla_status mla_query_project(const mla_shape* shape, int32_t d_cq, const void* x, int32_t n_frames,
                                     const void* w_dq, const void* w_uq, const void* w_qr, void* c_q, void* q_nope,
                                     void* q_r, void* stream) {
  return query_project_impl(shape, d_cq, x, n_frames, w_dq, w_uq, w_qr, c_q, q_nope, q_r, stream, true);
}

static mla_status output_project_impl(const mla_shape* shape, const void* o, int32_t n_frames, const void* w_o,
                                      void* u, void* stream, bool run) {
  mla_status st = check_shape(shape);
  if (st != MLA_OK) return st;
  if (!o || !w_o || !u) return MLA_ERR_NULL;
  if (!aligned16(o) || !aligned16(w_o) || !aligned16(u)) return MLA_ERR_ALIGN;
  if ((int64_t)shape->n_heads * shape->d_head > kMaxQueryLatent) return MLA_ERR_SHAPE;
  int64_t rows = 0;
  if ((st = check_projection_rows(shape, n_frames, &rows)) != MLA_OK) return st;
  if ((st = check_gemm_tiles(rows, shape->hidden)) != MLA_OK) return st;
  if (!run) return MLA_OK;
  return gemm(shape, o, w_o, nullptr, u, nullptr, rows, shape->hidden, shape->hidden, shape->n_heads * shape->d_head,
              (hipStream_t)stream);
}

MLA_API mla_status mla_output_project(const mla_shape* shape, const void* o, int32_t n_frames, const void* w_o,
                                      void* u, void* stream) {
  return output_project_impl(shape, o, n_frames, w_o, u, stream, true);
}

// ---------------------------------------------------------------- absorbed query path
MLA_API mla_status mla_query_absorb_weights(const mla_shape* shape, int32_t d_cq, const void* w_uq, const void* w_qr,
                                            const void* w_uk, void* w_qabs, void* stream) {
  mla_status st = check_shape(shape);
  if (st != MLA_OK) return st;
  if (!w_uq || !w_qr || !w_uk || !w_qabs) return MLA_ERR_NULL;
  if (!aligned16(w_uq) || !aligned16(w_qr) || !aligned16(w_uk) || !aligned16(w_qabs)) return MLA_ERR_ALIGN;
  if (d_cq < 8 || d_cq % 8 != 0 || d_cq > kMaxQueryLatent || shape->d_rope % 8 != 0) return MLA_ERR_SHAPE;
  if ((int64_t)shape->n_heads * qabs_dim(shape) > kMaxQueryLatent) return MLA_ERR_SHAPE;
  mla::QabsWeightParams p;
  p.w_uq = w_uq;
  p.w_qr = w_qr;
  p.w_uk = w_uk;
  p.w_qabs = w_qabs;
  p.H = shape->n_heads;
  p.d_head = shape->d_head;
  p.dc = shape->d_c;
  p.dr = shape->d_rope;
  p.kp = qabs_dim(shape);
  p.d_cq = d_cq;
  return from_hip(mla::launch_qabs_weights(shape->dtype, p, (hipStream_t)stream));
}

static mla_status query_project_absorbed_impl(const mla_shape* shape, int32_t d_cq, const void* x,
                                              int32_t q_frame_first, int32_t n_frames, const void* w_dq,
                                              const void* w_qabs, const float* rope_tables, int32_t rope_t_first,
                                              int32_t rope_n_t, void* c_q, void* q_abs, void* stream, bool run,
                                              bool cq_ready = false) {
  mla_status st = check_shape(shape);
  if (st != MLA_OK) return st;
  if (!x || !w_dq || !w_qabs || !c_q || !q_abs) return MLA_ERR_NULL;
  if (!aligned16(x) || !aligned16(w_dq) || !aligned16(w_qabs) || !aligned16(c_q) || !aligned16(q_abs))
    return MLA_ERR_ALIGN;
  if (d_cq < 8 || d_cq % 8 != 0 || d_cq > kMaxQueryLatent || shape->d_rope % 8 != 0) return MLA_ERR_SHAPE;
  const int n_abs = shape->n_heads * qabs_dim(shape);
  if ((int64_t)shape->n_heads * qabs_dim(shape) > kMaxQueryLatent) return MLA_ERR_SHAPE;
  if ((st = check_tables(shape, rope_tables, rope_t_first, rope_n_t)) != MLA_OK) return st;
  if ((st = check_query_args(shape, q_frame_first, n_frames)) != MLA_OK) return st;
  if (q_frame_first < rope_t_first || (int64_t)q_frame_first + n_frames > (int64_t)rope_t_first + rope_n_t)
    return MLA_ERR_RANGE;
  int64_t rows = 0;
  if ((st = check_projection_rows(shape, n_frames, &rows)) != MLA_OK) return st;
  if ((st = check_gemm_tiles(rows, d_cq)) != MLA_OK || (st = check_gemm_tiles(rows, n_abs)) != MLA_OK) return st;
  if (!run) return MLA_OK;
  hipStream_t s = (hipStream_t)stream;
  if (!cq_ready && (st = gemm(shape, x, w_dq, nullptr, c_q, nullptr, rows, d_cq, d_cq, shape->hidden, s)) != MLA_OK)
    return st;
  mla::GemmParams p{};
  p.a = c_q;
  p.b = w_qabs;
  p.c = q_abs;
  p.M = (int)rows;
  p.N = n_abs;
  p.K = d_cq;
  p.lda = d_cq;
  p.ldb = d_cq;
  p.ldc = n_abs;
  p.ldc2 = 0;
  p.n_split = n_abs;
  p.n_split2 = n_abs;
  p.qa.tables = rope_tables;
  p.qa.rl = rope_layout(shape, rope_t_first, rope_n_t);
  p.qa.kp = qabs_dim(shape);
  p.qa.dc = shape->d_c;
  p.qa.dr = shape->d_rope;
  p.qa.n_q = (int)(n_frames * tokens_per_frame(shape));
  p.qa.T = (int)tokens_per_frame(shape);
  p.qa.grid_x = shape->grid_x;
  p.qa.q_frame_first = q_frame_first;
  p.qa.qscale = scale_log2(shape);
  return from_hip(mla::launch_gemm_qabs(shape->dtype, p, mla::gemm_tile_rows(p.M, p.N, device_cus()), s));
}

MLA_API mla_status mla_query_project_absorbed(const mla_shape* shape, int32_t d_cq, const void* x,
                                              int32_t q_frame_first, int32_t n_frames, const void* w_dq,
                                              const void* w_qabs, const float* rope_tables, int32_t rope_t_first,
                                              int32_t rope_n_t, void* c_q, void* q_abs, void* stream) {
  return query_project_absorbed_impl(shape, d_cq, x, q_frame_first, n_frames, w_dq, w_qabs, rope_tables,
                                     rope_t_first, rope_n_t, c_q, q_abs, stream, true);
}

// ---------------------------------------------------------------- whole layer
namespace {

// Layer-step workspace: query latent, queries, the heads' outputs, then the
// attention side's own workspace.
struct LayerWs {
  size_t c_q, q_nope, q_r, o, attend, total;
};

LayerWs layer_ws_layout(const mla_shape* s, int d_cq, int n_frames) {
  const size_t rows = (size_t)s->batch * n_frames * tokens_per_frame(s);
  const size_t e = elt_size(s);
  LayerWs w;
  w.c_q = 0;
  w.q_nope = w.c_q + round256(rows * d_cq * e);
  w.q_r = w.q_nope + round256(rows * s->n_heads * s->d_head * e);
  w.o = w.q_r + round256(rows * s->n_heads * s->d_rope * e);
  w.attend = w.o + round256(rows * s->n_heads * s->d_head * e);
  w.total = w.attend + mla_chunk_attend_workspace_bytes(s, n_frames);
  return w;
}

}  // namespace

MLA_API size_t mla_layer_step_workspace_bytes(const mla_shape* shape, int32_t d_cq, int32_t n_frames) {
  if (check_shape(shape) != MLA_OK || check_query_args(shape, 0, n_frames) != MLA_OK || d_cq < 8 || d_cq % 8 != 0 ||
      d_cq > kMaxQueryLatent || mla_chunk_attend_workspace_bytes(shape, n_frames) == 0)
    return 0;
  return layer_ws_layout(shape, d_cq, n_frames).total;
}

MLA_API mla_status mla_layer_step(const mla_shape* shape, int32_t d_cq, const mla_layer_weights* weights,
                                  const void* x, int32_t frame_first, int32_t n_frames, void* cache,
                                  int32_t* slot_frame, const float* rope_tables, int32_t rope_t_first,
                                  int32_t rope_n_t, int32_t frame_causal, void* u, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  mla_status st = check_shape(shape);
  if (st != MLA_OK) return st;
  if (!weights || !workspace) return MLA_ERR_NULL;
  if (!aligned16(workspace)) return MLA_ERR_ALIGN;
  if (d_cq < 8 || d_cq % 8 != 0 || d_cq > kMaxQueryLatent) return MLA_ERR_SHAPE;
  if ((st = check_query_args(shape, frame_first, n_frames)) != MLA_OK) return st;
  const size_t need = mla_layer_step_workspace_bytes(shape, d_cq, n_frames);
  if (need == 0) return MLA_ERR_SHAPE;
  if (check_gemm_tiles((int64_t)shape->batch * n_frames * tokens_per_frame(shape), d_cq + shape->d_c + shape->d_rope) !=
      MLA_OK)
    return MLA_ERR_SHAPE;
  if (workspace_bytes < need) return MLA_ERR_WORKSPACE;
  const LayerWs w = layer_ws_layout(shape, d_cq, n_frames);
  char* ws = (char*)workspace;
  void *c_q = ws + w.c_q, *q_nope = ws + w.q_nope, *q_r = ws + w.q_r, *o = ws + w.o;
  const bool causal = frame_causal != 0;
  const mla_layer_weights& W = *weights;
  // the per-head form where mla_chunk_attend (or its frame-causal variant)
  // would take it (it needs the per-head queries, so the unfused query path)
  const bool heads = heads_preferred(shape, n_frames) && W.w_uq && W.w_qr && W.w_uk;
  if (W.w_qabs && !heads) {
    // fused query path: the query latent's product with the absorbed weights
    // is already the attention's query; workspace = [c_q | q_abs | o | o_lat, flash]
    const size_t rows = (size_t)shape->batch * n_frames * tokens_per_frame(shape) * shape->n_heads;
    char* q_abs = ws + w.q_nope;
    char* o2 = q_abs + round256(rows * qabs_dim(shape) * elt_size(shape));
    char* att = o2 + round256(rows * shape->d_head * elt_size(shape));
    if (att > ws + w.total) return MLA_ERR_WORKSPACE;  // cannot happen: the layout is smaller than the unfused one
    const size_t att_bytes = (size_t)(ws + w.total - att);
    for (int pass = 0; pass < 2; ++pass) {
      const bool run = pass == 1;
      // the query latent and the cache write in one pass over x, then the rest
      if ((st = cache_write_impl(shape, x, W.w_dkv, W.w_kr, frame_first, n_frames, cache, slot_frame, stream, false)) !=
          MLA_OK)
        return st;
      if (run && (st = gemm_query_latent_and_cache(shape, d_cq, x, W.w_dq, W.w_dkv, W.w_kr, frame_first, n_frames, c_q,
                                                   cache, slot_frame, (hipStream_t)stream)) != MLA_OK)
        return st;
      if ((st = query_project_absorbed_impl(shape, d_cq, x, frame_first, n_frames, W.w_dq, W.w_qabs, rope_tables,
                                            rope_t_first, rope_n_t, c_q, q_abs, stream, run, true)) != MLA_OK)
        return st;
      if ((st = attend_absorbed_impl(shape, q_abs, frame_first, n_frames, W.w_uv, cache, slot_frame, rope_tables,
                                     rope_t_first, rope_n_t, o2, att, att_bytes, stream, causal, run)) != MLA_OK)
        return st;
      if ((st = output_project_impl(shape, o2, n_frames, W.w_o, u, stream, run)) != MLA_OK) return st;
    }
    return MLA_OK;
  }
  // every part is validated before the first launch
  for (int pass = 0; pass < 2; ++pass) {
    const bool run = pass == 1;
    // the query latent and the cache write in one pass over x, then the rest
    if ((st = cache_write_impl(shape, x, W.w_dkv, W.w_kr, frame_first, n_frames, cache, slot_frame, stream, false)) !=
        MLA_OK)
      return st;
    if (run && (st = gemm_query_latent_and_cache(shape, d_cq, x, W.w_dq, W.w_dkv, W.w_kr, frame_first, n_frames, c_q,
                                                 cache, slot_frame, (hipStream_t)stream)) != MLA_OK)
      return st;
    if ((st = query_project_impl(shape, d_cq, x, n_frames, W.w_dq, W.w_uq, W.w_qr, c_q, q_nope, q_r, stream, run,
                                 true)) != MLA_OK)
      return st;
    if (heads) {
      st = chunk_attend_heads_impl(shape, q_nope, q_r, frame_first, n_frames, W.w_uk, W.w_uv, cache, slot_frame,
                                   rope_tables, rope_t_first, rope_n_t, o, ws + w.attend, w.total - w.attend, stream,
                                   run, causal);
    } else {
      st = chunk_attend_impl(shape, q_nope, q_r, frame_first, n_frames, W.w_uk, W.w_uv, cache, slot_frame, rope_tables,
                             rope_t_first, rope_n_t, o, ws + w.attend, w.total - w.attend, stream, causal, run);
    }
    if (st != MLA_OK) return st;
    if ((st = output_project_impl(shape, o, n_frames, W.w_o, u, stream, run)) != MLA_OK) return st;
  }
  return MLA_OK;
}
