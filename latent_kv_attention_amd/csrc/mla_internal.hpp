// Internal launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mla {

// Offsets (in floats) of the six RoPE tables inside one table buffer.
struct RopeLayout {
  int d_t, d_y, d_x;
  int t_first, n_t;
  int off_ct, off_st, off_cy, off_sy, off_cx, off_sx;
};

struct RopeTableParams {
  float* tables;
  RopeLayout rl;
  int grid_y, grid_x;
  double base;
  int total;  // number of (position, pair) entries over the three axes
};

struct CacheWriteParams {
  const void* x;       // [rows][hidden]
  const void* w_dkv;   // [d_c][hidden]
  const void* w_kr;    // [d_rope][hidden]
  void* cache;         // [B][W][T][d_c + d_rope]
  int32_t* slot_frame; // [B][W]
  int rows;            // B * n_frames * T
  int rows_per_b;      // n_frames * T
  int hidden, d_c, d_rope, W, T, frame_first, n_frames, batch;
};

struct AbsorbParams {
  const void* q_nope;  // [B*Nq][H][d_head]
  const void* q_r;     // [B*Nq][H][d_rope]
  const void* w_uk;    // [H][d_head][d_c]
  const float* tables;
  void* q_abs;         // [B*Nq][H][Q]
  RopeLayout rl;
  int rows;            // B * Nq
  int n_q, H, d_head, T, grid_x, q_frame_first;
  float qscale;        // softmax scale * log2(e)
};

// The attention work is a grid of units (row block, key tile) in
// row-block-major order. Row blocks come in classes of consecutive blocks
// (one class without the frame-causal mask; with it, class k holds the row
// blocks whose last row is a query of chunk frame k), and every row block of
// class k has nt[k] units, the key tiles of the window part its rows may see
// when the window is full (the frames up to its last row's). The first
// rb_whole row blocks (a multiple of G, all streams counted) are dealt whole
// in rounds: work-group g takes row block k G + g in round k. The units left,
// [u_rest, U), are shared by work-groups g < G' (grid_rest): g takes
// [u_rest + g R / G', u_rest + (g + 1) R / G'), R = U - u_rest; a row block
// that falls to several work-groups is finished by a merge pass over their
// partial results.
constexpr int kMaxUnitClasses = 64;
struct UnitClasses {
  int n;                          // classes
  int rb_end[kMaxUnitClasses];    // row block after the last of class k (within a stream)
  int nt[kMaxUnitClasses];        // units per row block of class k
  long long u0[kMaxUnitClasses];  // first unit of class k within a stream
  long long per_stream;           // units of one stream
};

// Row block rbg (over all streams) holding unit u: its first unit a and its
// unit count nt.
__host__ __device__ inline void locate_unit(const UnitClasses& c, int n_rb, long long u, long long& rbg,
                                            long long& a, int& nt) {
  const long long b = u / c.per_stream, v = u - b * c.per_stream;
  int k = 0;
  while (k + 1 < c.n && v >= c.u0[k + 1]) ++k;
  const int rb0 = k == 0 ? 0 : c.rb_end[k - 1];
  const long long r = (v - c.u0[k]) / c.nt[k];
  rbg = b * n_rb + rb0 + r;
  a = b * c.per_stream + c.u0[k] + r * c.nt[k];
  nt = c.nt[k];
}

// First unit and unit count of row block rbg (over all streams).
__host__ __device__ inline void row_block_units(const UnitClasses& c, int n_rb, long long rbg, long long& a,
                                                int& nt) {
  const long long b = rbg / n_rb;
  const int rb = (int)(rbg - b * n_rb);
  int k = 0;
  while (k + 1 < c.n && rb >= c.rb_end[k]) ++k;
  const int rb0 = k == 0 ? 0 : c.rb_end[k - 1];
  a = b * c.per_stream + c.u0[k] + (long long)(rb - rb0) * c.nt[k];
  nt = c.nt[k];
}

struct FlashParams {
  const void* q_abs;       // [B][Mb][Q]
  const void* cache;       // [B][W][T][d_c + d_rope]
  const int32_t* slot_frame;
  const float* tables;
  void* o_lat;             // [B][Mb][d_c]
  void* part_o;            // [G][2][rows per block][d_c] partial outputs o_g / l_g, element type of the
                           // cache (split row blocks only)
  float* part_l;           // [G][2][rows per block][2] (log2 of the piece's weight, status)
  void* krot;              // [B][W * T][d_rope] rotated kR of each stream's valid keys, in key order
  int* fallback_count;     // rows listed for the exact fallback
  int* fallback_rows;      // [B * Mb]
  RopeLayout rl;
  int Mb;                  // Nq * H
  int W, T, grid_y, grid_x, batch;
  float inv_T, inv_grid_x; // 1/T and 1/grid_x (key index -> slot, row, column)
  int n_rb, nt_max;        // row blocks per stream, key tiles of a full window
  int H, q_frame_first;    // heads; first query frame (frame-causal variant)
  long long units;         // all units: batch * classes.per_stream
  UnitClasses classes;
  int grid;                // G, work-groups of the attention kernel
  long long rb_whole;      // row blocks dealt whole in rounds (a multiple of G)
  long long u_rest;        // first unit after them
  int grid_rest;           // work-groups sharing the units from u_rest on
  float scale_log2;        // softmax scale * log2(e)
  double rope_base;        // RoPE base (the keys' temporal angles are formed per call)
};

constexpr int kFallbackBlocks = 64;
// At most this many work-groups share one row block of the attention kernel
// (the host caps its work-group count at (kMaxMergePieces - 1) row blocks'
// worth, which bounds the pieces of a row block by kMaxMergePieces).
constexpr int kMaxMergePieces = 64;
// Limit of the attention kernel: keys per window (index arithmetic in float).
constexpr int kMaxWindowKeys = 1 << 22;

struct UpVParams {
  const void* o_lat;  // [B*Nq][H][d_c]
  const void* w_uv;   // [H][d_head][d_c]
  void* out;          // [B*Nq][H][d_head]
  int rows, H, d_head;
};

// Per-head form of the attention: keys and values of every head are
// reconstructed from the latent for the window once per call, then a
// standard two-part-score attention runs per head.
struct HeadsParams {
  const void* q_nope;      // [B][Nq][H][d_head]
  const void* q_r;         // [B][Nq][H][d_rope], unrotated
  const void* w_uk;        // [H][d_head][d_c]
  const void* w_uv;        // [H][d_head][d_c]
  const void* cache;       // [B][W][T][d_c + d_rope]
  const int32_t* slot_frame;
  const float* tables;
  void* out;               // [B][Nq][H][d_head]
  void* q_cat;             // [B][H][Nq][d_head + d_rope]: [q_nope | R(p) q_r] * scale * log2 e
  void* k_exp;             // [B][H][W * T][d_head]: W_uk[h] c_j of each valid key j, in key order
  void* v_exp;             // [B][H][W * T][d_head]: W_uv[h] c_j
  const void* krot;        // [B][W * T][d_rope]: rotated kR (the rotation pass of the latent form)
  int* fallback_count;     // rows listed for the exact fallback
  int* fallback_rows;      // [B * H * Nq], as (b * H + h) * Nq + i
  void* part_o;            // [G][2][rows per block][d_head] partial outputs o_g / l_g (split row blocks only)
  float* part_l;           // [G][2][rows per block][2] (log2 of the piece's weight, status)
  RopeLayout rl;
  int batch, H, Nq, T, W, grid_x, q_frame_first;
  int n_rb, nt_max;        // row blocks of kHeadsRowsPerBlock tokens per (stream, head); key tiles of a full window
  long long units;         // all units: batch * H * classes.per_stream
  UnitClasses classes;     // per (stream, head): row-block classes and their unit counts
  int grid;                // G, work-groups of the attention kernel
  long long rb_whole;      // row blocks dealt whole in rounds (a multiple of G)
  long long u_rest;        // first unit after them
  int grid_rest;           // work-groups sharing the units from u_rest on
  float qscale;            // softmax scale * log2(e)
};

// C[M][N] = A[M][K] B[N][K]^T (rows of B are output features), fp32
// accumulation, C in the operands' type. Features n >= n_split take their
// weight row from B2 (row n - n_split) and land in C2 (column n - n_split,
// row stride ldc2); n_split = N for one part. K, N, n_split and all strides
// multiples of 8; pointers 16-byte aligned.
// Epilogue of the absorbed-query product (GemmParams::qabs): the output row of
// a token is its absorbed queries [H][kp], head h = [dc latent | dr
// positional | zero pad]; the positional part is rotated by 3D-RoPE at the
// token's (t, y, x) and every value is multiplied by qscale before the one
// rounding to the element type.
struct GemmQabs {
  const float* tables;
  RopeLayout rl;
  int kp, dc, dr;
  int n_q, T, grid_x, q_frame_first;  // tokens per stream, per frame; frame of token 0
  float qscale;                       // softmax scale * log2(e)
};

// Ring epilogue of a product whose second output part is the cache write:
// token row r (stream b = r / rows_per_b, chunk token t = r % rows_per_b) of
// part 2 goes to cache row (b W + (frame_first + t / T) mod W) T + t mod T
// (row stride ldc2 = d_c + d_rope), and slot_frame[b][f mod W] = f is set for
// every written frame f.
struct GemmRing {
  int32_t* slot_frame;  // nullptr: part 2 is a plain matrix
  int rows_per_b, T, W, frame_first, n_frames, batch;
};

struct GemmParams {
  const void* a;
  const void* b;
  const void* b2;
  const void* b3;
  void* c;
  void* c2;
  // features n < n_split: weight b row n, output c column n; n_split <= n <
  // n_split2: weight b2 row n - n_split; n >= n_split2: weight b3 row
  // n - n_split2; both of the last two land in c2 column n - n_split
  int M, N, K, lda, ldb, ldc, ldc2, n_split, n_split2;
  int tiles_n, n_logical, per_xcd;  // filled by the launcher
  GemmQabs qa;                      // used only by the absorbed-query launch
  GemmRing ring;                    // used only by the ring launch
};

// Absorbed query weight of each head: w_qabs[h][j][:] = (W_uk[h]^T W_uq[h])[j][:]
// for j < dc, W_qr[h][j - dc][:] for dc <= j < dc + dr, zero up to kp.
struct QabsWeightParams {
  const void* w_uq;  // [H][d_head][d_cq]
  const void* w_qr;  // [H][dr][d_cq]
  const void* w_uk;  // [H][d_head][dc]
  void* w_qabs;      // [H][kp][d_cq]
  int H, d_head, dc, dr, kp, d_cq;
};

hipError_t launch_rope_tables(const RopeTableParams& p, hipStream_t s);
hipError_t launch_cache_write(int dtype, int d_c, int d_rope, const CacheWriteParams& p, hipStream_t s);
hipError_t launch_absorb_q(int dtype, int d_c, int d_rope, const AbsorbParams& p, hipStream_t s);
// causal: the frame-causal variant (a query of frame f sees keys of frames <= f)
hipError_t launch_flash(int dtype, int d_c, int d_rope, const FlashParams& p, bool split, bool causal,
                        hipStream_t s);
hipError_t launch_up_v(int dtype, int d_c, int d_rope, const UpVParams& p, hipStream_t s);
// the rotation pass of the attention kernel alone (rotated kR of the window
// into p.krot, fallback count cleared)
hipError_t launch_rope_window(int dtype, int d_c, int d_rope, const FlashParams& p, hipStream_t s);
// Query tokens per row block of the per-head attention kernel (8 waves of
// 48 tokens of one head).
constexpr int kHeadsRowsPerBlock = 384;
bool heads_supported(int dtype, int d_c, int d_rope, int d_head);
int heads_tile_keys(int d_head, int d_rope);  // keys per tile of the per-head attention kernel
// causal: the frame-causal variant (a query of frame f sees keys of frames <= f)
hipError_t launch_heads(int d_c, int d_rope, int d_head, const HeadsParams& p, bool split, bool causal,
                        hipStream_t s);
// tile of the projection GEMM (128 x 128 or 64 x 64, given by its rows) for
// a problem of M x N outputs on n_cu compute units
int gemm_tile_rows(int M, int N, int n_cu);
hipError_t launch_gemm_nt(int dtype, const GemmParams& p, int tile_rows, hipStream_t s);
// the same product with the absorbed-query epilogue (p.qa)
hipError_t launch_gemm_qabs(int dtype, const GemmParams& p, int tile_rows, hipStream_t s);
// the same product with part 2 scattered into the ring cache (p.ring)
hipError_t launch_gemm_ring(int dtype, const GemmParams& p, int tile_rows, hipStream_t s);
hipError_t launch_qabs_weights(int dtype, const QabsWeightParams& p, hipStream_t s);

}  // namespace mla
