// Per-head form of the chunk attention. hyper.ai summary of VideoMLA,
// Method section: the cache holds only the shared latent c_j and the
// positional key kR_j, and the per-head keys and values are reconstructed
// from c_j when they are needed. This file reconstructs them for the whole
// window once per call,
//   k_exp[h][j] = W_uk[h] c_j,   v_exp[h][j] = W_uv[h] c_j   (j in key order),
// and then runs, per head, attention with the two-part score
//   s_ij = scale * (q_nope_ih . k_exp[h][j] + R(p_i) qR_ih . R(p_j) kR_j)
//   out_ih = sum_j softmax_j(s_ij) v_exp[h][j].
// The attention does 2 Nq Nk H (d_head + d_rope + d_head) products against
// the latent form's 2 Nq Nk H (d_c + d_rope + d_c); the expansion adds
// 4 Nk H d_head d_c products and writes 4 Nk H d_head bytes (bf16).
//
// Attention layout (bf16): a row block is 384 query tokens of one head (8
// waves x 48 rows, two waves per SIMD: each staged key and value fragment
// feeds three row blocks' products); one work-group per compute unit
// takes an equal share of the (row block, key tile) units, and row blocks
// shared by several work-groups are merged afterwards. Key tiles of 128 keys are staged in LDS, double buffered, with
// direct global->LDS loads from three contiguous row sets: k_exp (rows 272
// bytes apart), the rotated kR (packed, 16-byte units XOR-swizzled by key)
// and v_exp (rows 288 bytes apart, the stride at which the transposing reads
// of the value product do not conflict). Scores are formed transposed,
// S^T = K Q^T, so the probabilities land in the operand layout of
// O^T = V^T P^T; the softmax uses a fixed per-row reference (the maximum of
// the first 32 keys' scores) and lists rows whose sum leaves [2^-100, 2^100]
// for an exact two-pass kernel, as the latent form does; the frame-causal
// variant walks each row's visible prefix of the window.
#include <type_traits>

#include "mla_common.hpp"
#include "mla_internal.hpp"
#include "rope_device.hpp"

namespace mla {

namespace {
constexpr int kSlots = 64;
constexpr float kHeadsSumLimit = 0x1p100f;
constexpr float kHeadsSumMin = 0x1p-100f;
constexpr int kExpWaves = 8;
constexpr int kExpKeys = kExpWaves * 64;  // keys per expansion work-group

__device__ __forceinline__ int opaque_h(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

__device__ __forceinline__ void store4_bf16(bf16* dst, float a, float b, float c, float d) {
  const uint32_t w0 = (uint32_t)__builtin_bit_cast(uint16_t, (bf16)a) |
                      ((uint32_t)__builtin_bit_cast(uint16_t, (bf16)b) << 16);
  const uint32_t w1 = (uint32_t)__builtin_bit_cast(uint16_t, (bf16)c) |
                      ((uint32_t)__builtin_bit_cast(uint16_t, (bf16)d) << 16);
  *reinterpret_cast<u32x2*>(dst) = u32x2{w0, w1};
}

// valid slots of stream b in key order (by frame, window_rank; wave 0); fills LDS
__device__ __forceinline__ void slot_ranks(const HeadsParams& p, int b, int lane, int* slot_of, int* n_valid) {
  const int f = lane < p.W ? p.slot_frame[b * p.W + lane] : -1;
  const int rank = window_rank(f, lane);  // key order of the rotated kR (rope_window_kernel)
  if (f >= 0) slot_of[rank] = lane;
  const unsigned long long mask = __ballot(f >= 0);
  if (lane == 0) *n_valid = __popcll(mask);
}
}  // namespace

// ---------------------------------------------------------------- expansion
// k_exp / v_exp rows of 512 keys of one head of one stream. Both weight
// matrices of the head are staged in LDS; each wave takes 64 keys and
// computes out^T = W c^T in 16 x 16 blocks. The staged weight rows are
// in expand_pos order, so the blocks 2m and 2m + 1 leave a lane with
// outputs 32 m + 8 lg .. 32 m + 8 lg + 7 of one key (lg = lane / 16),
// stored as one 16-byte piece; the four lanes of a key write 64 contiguous
// bytes.
template <int DC, int DR, int DH>
__global__ __launch_bounds__(512) void expand_kv_kernel(HeadsParams p) {
  constexpr int LSW = DC + 16;  // LDS row stride of the staged weights (elements)
  constexpr int NKC = DC / 32;
  constexpr int NNB = DH / 16;
  constexpr int CPW = DC / 8;                  // 16-byte pieces per weight row
  constexpr int WPT = (2 * DH * CPW + 511) / 512;  // pieces per thread
  static_assert(DH % 32 == 0, "pairs of 16-row blocks");
  __shared__ __attribute__((aligned(16))) bf16 wl[2 * DH * LSW];
  __shared__ int slot_of[kSlots];
  __shared__ int n_valid_sh;
  const int h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  if (wave == 0) slot_ranks(p, b, lane, slot_of, &n_valid_sh);
  // every weight piece of this thread requested before any is written to LDS
  bf16x8 wst[WPT];
#pragma unroll
  for (int i = 0; i < WPT; ++i) {
    const int e = tid + 512 * i;
    if (e < 2 * DH * CPW) {
      const int r = e / CPW, c8 = (e - r * CPW) * 8;
      wst[i] = load8<bf16>((const bf16*)(r < DH ? p.w_uk : p.w_uv) + ((size_t)h * DH + (r < DH ? r : r - DH)) * DC + c8);
    }
  }
  __syncthreads();  // slot ranks
  const int n_keys = n_valid_sh * p.T;
  if (blockIdx.x * kExpKeys >= n_keys) return;  // the whole work-group past the window
  const int v0 = blockIdx.x * kExpKeys + wave * 64;

  // c of this wave's 64 keys (keys past the window alias the last key; their
  // outputs are not stored), as the B operand: key li of block mb, dims
  // kc * 32 + lg * 8; requested before the weights land in LDS
  const bf16* cache_b = (const bf16*)p.cache + (size_t)b * p.W * p.T * (DC + DR);
  bf16x8 cb[4][NKC];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int v = min(v0 + mb * 16 + li, n_keys - 1);
    const int rank = v / p.T, tok = v - rank * p.T;
    const bf16* row = cache_b + ((size_t)slot_of[rank] * p.T + tok) * (DC + DR);
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) cb[mb][kc] = load8<bf16>(row + kc * 32 + lg * 8);
  }
#pragma unroll
  for (int i = 0; i < WPT; ++i) {
    const int e = tid + 512 * i;
    if (e < 2 * DH * CPW) {
      const int r = e / CPW, c8 = (e - r * CPW) * 8;
      const int m = r < DH ? 0 : 1, d = r - m * DH;
      store8<bf16>(wl + (m * DH + expand_pos(d)) * LSW + c8, wst[i]);
    }
  }
  __syncthreads();
  if (v0 >= n_keys) return;

  const size_t head_rows = (size_t)(b * p.H + h) * p.W * p.T;
  const bool full = v0 + 64 <= n_keys;
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    bf16* dst = (bf16*)(which == 0 ? p.k_exp : p.v_exp) + head_rows * DH;
#pragma unroll 1
    for (int m = 0; m < NNB / 2; ++m) {
      f32x4 acc[2][4] = {};
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int nb = 2 * m + half;
        bf16x8 a[NKC];
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) a[kc] = lds_load8<bf16>(wl + (which * DH + nb * 16 + li) * LSW + kc * 32 + lg * 8);
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
          for (int mb = 0; mb < 4; ++mb) acc[half][mb] = mma16(a[kc], cb[mb][kc], acc[half][mb]);
      }
      // lane: outputs 32 m + 8 lg + (0..7) of key v0 + 16 mb + li
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const int v = v0 + mb * 16 + li;
        float f[8] = {acc[0][mb][0], acc[0][mb][1], acc[0][mb][2], acc[0][mb][3],
                      acc[1][mb][0], acc[1][mb][1], acc[1][mb][2], acc[1][mb][3]};
        if (full || v < n_keys) store8<bf16>(dst + (size_t)v * DH + m * 32 + lg * 8, pack8<bf16>(f));
      }
    }
  }
}

// ---------------------------------------------------------------- queries
// q_cat[b][h][i] = qscale * [q_nope | R(t, y, x) qR] for the chunk's tokens;
// one thread per 8-element piece.
template <int DH, int DR>
__global__ __launch_bounds__(256) void heads_qcat_kernel(HeadsParams p) {
  constexpr int QP = DH + DR, NC = QP / 8;
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long rows = (long long)p.batch * p.Nq * p.H;
  if (e >= rows * NC) return;
  const long long row = e / NC;  // (b, i, h) in the order of q_nope
  const int c = (int)(e - row * NC);
  const int h = (int)(row % p.H);
  const long long bi = row / p.H;
  const int i = (int)(bi % p.Nq), b = (int)(bi / p.Nq);
  float f[8];
  if (c < DH / 8) {
    unpack8<bf16>(load8<bf16>((const bf16*)p.q_nope + row * DH + c * 8), f);
#pragma unroll
    for (int k = 0; k < 8; ++k) f[k] *= p.qscale;
  } else {
    const int e0 = c * 8 - DH;  // first q_r element of the piece
    unpack8<bf16>(load8<bf16>((const bf16*)p.q_r + row * DR + e0), f);
    const int t = p.q_frame_first + i / p.T, tok = i % p.T;
    const int y = tok / p.grid_x, x = tok - y * p.grid_x;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float cs, sn;
      rope_cos_sin(p.rl, p.tables, e0 / 2 + k, t, y, x, cs, sn);
      rotate_pair(f[2 * k], f[2 * k + 1], cs, sn);
      f[2 * k] *= p.qscale;
      f[2 * k + 1] *= p.qscale;
    }
  }
  store8<bf16>((bf16*)p.q_cat + (((size_t)b * p.H + h) * p.Nq + i) * QP + c * 8, pack8<bf16>(f));
}

// ---------------------------------------------------------------- attention
template <int DH, int DR>
struct HeadsTile {
  static constexpr int kWaves = 8, kThreads = 512, kNMB = 3;
  static constexpr int kRowsWave = kNMB * 16, kRowsBlock = kWaves * kRowsWave;
  static_assert(kRowsBlock == kHeadsRowsPerBlock, "the host plans row blocks of this size");
  static constexpr int QP = DH + DR;           // contraction width of QK
  static constexpr int NKC = QP / 32, NKCH = DH / 32, NDB = DH / 16;
  static constexpr int LSK = DH + 8;           // k rows (elements): 16 rows of a QK read hit 16 bank groups
  static constexpr int LSV = DH + 16;          // v rows: four rows of a transposing read hit disjoint banks
  static constexpr int CPRK = LSK / 8, CPRV = LSV / 8, CH = DH / 8;
  static constexpr int U8 = DR / 8;            // 16-byte kR units per key
  // kR unit u of key n sits at kr_slot(n, u), chosen by measuring the bank
  // conflicts of the QK reads per layout: with 64-byte keys (4 units) keys 8
  // apart take disjoint unit pairs (XOR by (n / 4) mod 4 conflicted 2-way),
  // with 128-byte keys XOR by (n / 2) mod 8 is conflict-free
  static constexpr int KR_SH = U8 >= 16 ? 0 : U8 == 8 ? 1 : U8 == 4 ? 2 : U8 == 2 ? 3 : 4;
  __host__ __device__ static constexpr int kr_slot(int n, int u) {
    return U8 == 4 ? (u ^ (((n >> 3) & 1) * 2)) : U8 > 1 && U8 <= 16 ? (u ^ ((n >> KR_SH) & (U8 - 1))) : u;
  }
  static constexpr int instr(int keys, int chunks_per_key) { return (keys * chunks_per_key + 63) / 64; }
  static constexpr int buf_bytes(int keys) {
    return (instr(keys, CPRK) + instr(keys, CPRV) + instr(keys, U8)) * 64 * 16;
  }
  static constexpr int kBN = 2 * buf_bytes(128) <= 160 * 1024 - 1024 ? 128 : 64;  // keys per tile
  static constexpr int NKC2 = kBN / 32;
  static constexpr int K_INSTR = instr(kBN, CPRK), V_INSTR = instr(kBN, CPRV), R_INSTR = instr(kBN, U8);
  static constexpr int K_IW = (K_INSTR + kWaves - 1) / kWaves;
  static constexpr int V_IW = (V_INSTR + kWaves - 1) / kWaves;
  static constexpr int R_IW = (R_INSTR + kWaves - 1) / kWaves;
  static constexpr int K_ELEMS = K_INSTR * 64 * 8, V_ELEMS = V_INSTR * 64 * 8, R_ELEMS = R_INSTR * 64 * 8;
  static_assert(DH % 32 == 0 && DR % 32 == 0 && (U8 & (U8 - 1)) == 0, "whole 32-wide contraction blocks");
};

// CAUSAL: the frame-causal variant (a query of frame f attends only keys of
// frames <= f). Keys are in frame order, so the keys a row sees are a prefix
// of the window; as in the latent form, only the units a row block may see
// are dealt out (classes of row blocks), the tiles not seen whole by every
// row of a block are visited first through the limited tile body (keys past
// each row's prefix weigh zero), the rest with the plain body.
template <int DH, int DR, bool CAUSAL>
__global__ __launch_bounds__(512, 1) void heads_flash_kernel(HeadsParams p) {
  typedef HeadsTile<DH, DR> F;
  constexpr int kBN = F::kBN, kNMB = F::kNMB, kWaves = F::kWaves, NKC2 = F::NKC2;
  // one separately declared array per buffer and region, so every LDS access
  // has a compile-time array and the compiler does not wait for the
  // prefetch of the other buffer before reading the current one
  __shared__ __attribute__((aligned(16))) bf16 k0[F::K_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16 k1[F::K_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16 v0[F::V_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16 v1[F::V_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16 r0[F::R_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16 r1[F::R_ELEMS];
  __shared__ int n_valid_sh;
  __shared__ int frame_of[CAUSAL ? kSlots : 1];  // frame held by the r-th valid slot
  // frame-causal: end of each row's visible key prefix (in LDS, not in
  // registers: the tile body keeps its load descriptors resident)
  __shared__ int vis_sh[CAUSAL ? F::kRowsBlock : 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  // direct-load slots: instruction k of the wave fills chunks [64 i, 64 i + 64)
  // of a region, i = wave + kWaves k; packed (key << 16) | byte offset in the
  // key's source row, or -1 for padding chunks and spare instructions
  int kpk[F::K_IW], vpk[F::V_IW], rpk[F::R_IW];
#pragma unroll
  for (int k = 0; k < F::K_IW; ++k) {
    const int ins = wave + kWaves * k, q = ins * 64 + lane, n = q / F::CPRK, c = q - n * F::CPRK;
    kpk[k] = (ins < F::K_INSTR && n < kBN && c < F::CH) ? (n << 16) | (c * 16) : -1;
  }
#pragma unroll
  for (int k = 0; k < F::V_IW; ++k) {
    const int ins = wave + kWaves * k, q = ins * 64 + lane, n = q / F::CPRV, c = q - n * F::CPRV;
    vpk[k] = (ins < F::V_INSTR && n < kBN && c < F::CH) ? (n << 16) | (c * 16) : -1;
  }
#pragma unroll
  for (int k = 0; k < F::R_IW; ++k) {
    const int ins = wave + kWaves * k, q = ins * 64 + lane, n = q / F::U8, us = q - n * F::U8;
    rpk[k] = (ins < F::R_INSTR && n < kBN) ? (n << 16) | (F::kr_slot(n, us) * 16) : -1;
  }

  typedef bf16x8 v8;
  typedef f32x4 sblk[2][kNMB];
  typedef std::integral_constant<int, 0> B0;
  typedef std::integral_constant<int, 1> B1;

  // Work-group g (logical index, XCD-major) first takes its whole row
  // blocks, one per round (row block k G + g: the work-groups of an XCD hold
  // consecutive row blocks, mostly of one (stream, head), and walk its keys
  // in step, sharing them through the L2), then its range of the remaining
  // units, [u_rest + g R / G', u_rest + (g + 1) R / G'), as segments of at
  // most one row block each, last to first (so most work-groups read the
  // same few key tiles at any moment). A segment covering its whole row
  // block writes the output; a partial one writes (output / sum, reference,
  // sum) to slot 0 (the work-group's first segment of the range) or 1 (its
  // last) for the merge pass.
  const long long G = p.grid;
  const int g = xcd_major(blockIdx.x, p.grid);
  const long long rounds = p.rb_whole / G;
  const long long rest = p.units - p.u_rest;
  const long long u_first = g < p.grid_rest ? p.u_rest + (long long)g * rest / p.grid_rest : p.units;
  const long long u_last = g < p.grid_rest ? p.u_rest + ((long long)g + 1) * rest / p.grid_rest : p.units;
  long long round = 0;
  for (long long u = u_last;;) {
    long long rbg, ua;  // row block over all (stream, head) pairs, its first unit
    int nt;             // its unit count
    int j0, j1;
    bool first_seg;
    if (round < rounds) {
      rbg = round * G + g;
      ++round;
      row_block_units(p.classes, p.n_rb, rbg, ua, nt);
      j0 = 0;
      j1 = nt;
      first_seg = false;
    } else {
      if (u <= u_first) break;
      locate_unit(p.classes, p.n_rb, u - 1, rbg, ua, nt);
      const long long seg0 = max(u_first, ua);
      j0 = (int)(seg0 - ua);
      j1 = (int)(u - ua);
      first_seg = seg0 == u_first;
      u = seg0;
    }
    const bool whole = j0 == 0 && j1 == nt;
    const int bh = (int)(rbg / p.n_rb), rb = (int)(rbg - (long long)bh * p.n_rb);  // bh = b * H + h
    const int h = bh % p.H, b = bh / p.H;
    __syncthreads();  // LDS of the previous segment is no longer read
    if (wave == 0) {
      const int f = lane < p.W ? p.slot_frame[b * p.W + lane] : -1;
      if constexpr (CAUSAL) {
        const int rank = window_rank(f, lane);
        if (f >= 0) frame_of[rank] = f;
      }
      const unsigned long long mask = __ballot(f >= 0);
      if (lane == 0) n_valid_sh = __popcll(mask);
    }
    __syncthreads();
    const int n_keys = n_valid_sh * p.T;
    const int tok_wave = rb * F::kRowsBlock + wave * F::kRowsWave;
    // Frame-causal variant: the end of the visible prefix of each row of the
    // wave (vis_sh, read through vis_end: T times the valid slots whose frame
    // is at most the row's), of the block's first row (vis_lo: every row sees
    // the keys before it) and of its last row (n_keys_rb: the keys the block
    // visits). A wave writes and reads only its own rows' entries.
    int vis_lo = n_keys, n_keys_rb = n_keys;
    if constexpr (CAUSAL) {
      auto visible_keys = [&](int qf) {
        int n = 0;
        for (int r = 0; r < n_valid_sh; ++r) n += frame_of[r] <= qf ? 1 : 0;
        return n * p.T;
      };
#pragma unroll
      for (int mb = 0; mb < kNMB; ++mb) {
        const int tok = tok_wave + mb * 16 + li;
        if (lg == 0)
          vis_sh[wave * F::kRowsWave + mb * 16 + li] = tok < p.Nq ? visible_keys(p.q_frame_first + tok / p.T) : n_keys;
      }
      const int t_first = rb * F::kRowsBlock, t_last = min(t_first + F::kRowsBlock, p.Nq) - 1;
      vis_lo = visible_keys(p.q_frame_first + t_first / p.T);
      n_keys_rb = visible_keys(p.q_frame_first + t_last / p.T);
    }
    // visible prefix of the lane's row mb (the window's keys without the mask)
    auto vis_end = [&](int mb) { return CAUSAL ? vis_sh[wave * F::kRowsWave + mb * 16 + li] : n_keys; };
    const int n_tiles = (n_keys_rb + kBN - 1) / kBN;
    // this segment's share of the row block's tiles (units map onto the
    // tiles of a full window; a partly filled window scales proportionally)
    const int tile_begin = (int)((long long)j0 * n_tiles / nt);
    const int tile_end = (int)((long long)j1 * n_tiles / nt);
    const int n_visit = max(0, tile_end - tile_begin);
    // Positions 0 .. n_lim - 1 visit the range's last tiles, last first,
    // through the limited body (past the window for the ragged last tile;
    // past the row's prefix under the frame-causal mask: the tiles not seen
    // whole by every row of the block, an odd count where the range allows,
    // so the plain positions start on the same tile buffer).
    int n_lim = n_visit > 0 ? 1 : 0;
    if constexpr (CAUSAL) {
      if (n_visit > 0) {
        int m = max(1, tile_end - max(tile_begin, vis_lo / kBN));
        if (m % 2 == 0) m = min(m + 1, n_visit);
        n_lim = m;
      }
    }

    // queries of this wave (B operand of S^T = K Q^T), kept in registers
    const bf16* qb = (const bf16*)p.q_cat + (size_t)bh * p.Nq * F::QP;
    v8 qf[kNMB][F::NKC];
#pragma unroll
    for (int mb = 0; mb < kNMB; ++mb) {
      const int tok = tok_wave + mb * 16 + li;
#pragma unroll
      for (int kc = 0; kc < F::NKC; ++kc)
        qf[mb][kc] = tok < p.Nq ? load8<bf16>(qb + (size_t)tok * F::QP + kc * 32 + lg * 8) : zero8<bf16>();
    }
    f32x4 negref[kNMB];
    f32x4 o[F::NDB][kNMB];
    float l_run[kNMB];
#pragma unroll
    for (int mb = 0; mb < kNMB; ++mb) {
      negref[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
      l_run[mb] = 0.f;
#pragma unroll
      for (int db = 0; db < F::NDB; ++db) o[db][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const size_t head_rows = (size_t)bh * p.W * p.T;
    const char* kb_src = (const char*)((const bf16*)p.k_exp + head_rows * DH);
    const char* vb_src = (const char*)((const bf16*)p.v_exp + head_rows * DH);
    const char* rb_src = (const char*)((const bf16*)p.krot + (size_t)b * p.W * p.T * DR);

    // buffer resources of the head's expanded keys and values and the
    // stream's rotated kR: the buffer form of the direct loads counts its LDS
    // writes on the vector-memory counter alone, so the operand reads keep
    // exact partial waits while the next tile's loads are in flight
    const __amdgpu_buffer_rsrc_t k_rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)kb_src, 0, (int)((size_t)p.W * p.T * DH * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t v_rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)vb_src, 0, (int)((size_t)p.W * p.T * DH * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t r_rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)rb_src, 0, (int)((size_t)p.W * p.T * DR * 2), 0x00020000);
    auto tile_of = [&](int pos) { return pos < n_lim ? tile_end - 1 - pos : tile_begin + pos - n_lim; };
    auto issue = [&](int pos, bf16* kt, bf16* vt, bf16* rt) {
      const int kbase = tile_of(pos) * kBN;
#pragma unroll
      for (int k = 0; k < F::K_IW; ++k) {
        const int pk = opaque_h(kpk[k]);
        if (pk >= 0) {
          const int v = min(kbase + (pk >> 16), n_keys - 1);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(k_rs, (MLA_LDS void*)(MLA_LDS bf16*)(kt + (wave + kWaves * k) * 64 * 8), 16,
                                                   (unsigned)(v * DH * 2 + (pk & 0xffff)), 0, 0, 0);
        }
      }
#pragma unroll
      for (int k = 0; k < F::V_IW; ++k) {
        const int pk = opaque_h(vpk[k]);
        if (pk >= 0) {
          const int v = min(kbase + (pk >> 16), n_keys - 1);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(v_rs, (MLA_LDS void*)(MLA_LDS bf16*)(vt + (wave + kWaves * k) * 64 * 8), 16,
                                                   (unsigned)(v * DH * 2 + (pk & 0xffff)), 0, 0, 0);
        }
      }
#pragma unroll
      for (int k = 0; k < F::R_IW; ++k) {
        const int pk = opaque_h(rpk[k]);
        if (pk >= 0) {
          const int v = min(kbase + (pk >> 16), n_keys - 1);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(r_rs, (MLA_LDS void*)(MLA_LDS bf16*)(rt + (wave + kWaves * k) * 64 * 8), 16,
                                                   (unsigned)(v * DR * 2 + (pk & 0xffff)), 0, 0, 0);
        }
      }
    };
    auto scores = [&](const bf16* kt, const bf16* rt, int half, sblk& s, const f32x4 (&seed)[kNMB]) {
#pragma unroll
      for (int kc = 0; kc < F::NKC; ++kc) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int row = (half * 2 + kb) * 16 + li, dim = kc * 32 + lg * 8;
          const v8 a = kc < F::NKCH ? lds_load8<bf16>(kt + row * F::LSK + dim)
                                    : lds_load8<bf16>(rt + row * DR + F::kr_slot(row, (dim - DH) / 8) * 8);
#pragma unroll
          for (int mb = 0; mb < kNMB; ++mb) s[kb][mb] = mma16(a, qf[mb][kc], kc == 0 ? seed[mb] : s[kb][mb]);
        }
      }
    };
    // limited body: key kfirst + 4 lg + 16 kb + i is kept when 16 kb + i <
    // lim, the limit being the row's visible prefix under the frame-causal
    // mask, else the window's end (the lane offset recomputed here)
    auto probs = [&](const sblk& s, v8 (&pb)[kNMB], int kfirst, auto limited_c) {
      constexpr bool LIMITED = decltype(limited_c)::value;
#pragma unroll
      for (int mb = 0; mb < kNMB; ++mb) {
        float f8[8];
        int lim = 0;
        if constexpr (LIMITED) lim = vis_end(mb) - kfirst - 4 * opaque_h(lg);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float e = fast_exp2(s[kb][mb][i]);
            if constexpr (LIMITED) e = kb * 16 + i < lim ? e : 0.f;
            f8[kb * 4 + i] = e;
            l_run[mb] += e;
          }
        pb[mb] = pack8<bf16>(f8);
      }
    };
    // The tile body's products with their operand reads run ahead: score
    // operands DQ contraction steps, value operands DV d-blocks (scheduling
    // barriers keep each read that far ahead of its product).
    auto scores_ahead = [&](const bf16* kt, const bf16* rt, int half, sblk& s) {
      // one contraction step ahead (three ahead measured 1% slower at d_rope 32;
      // the wider positional part leaves no registers for more)
      constexpr int DQ = 1;
      v8 ka[DQ + 1][2];
      auto kop = [&](int kc, int kb) -> v8 {
        const int row = (half * 2 + kb) * 16 + li, dim = kc * 32 + lg * 8;
        return kc < F::NKCH ? lds_load8<bf16>(kt + row * F::LSK + dim)
                            : lds_load8<bf16>(rt + row * DR + F::kr_slot(row, (dim - DH) / 8) * 8);
      };
#pragma unroll
      for (int d = 0; d < DQ; ++d)
        if (d < F::NKC) {
          ka[d][0] = kop(d, 0);
          ka[d][1] = kop(d, 1);
        }
#pragma unroll
      for (int kc = 0; kc < F::NKC; ++kc) {
        if (kc + DQ < F::NKC) {
          ka[(kc + DQ) % (DQ + 1)][0] = kop(kc + DQ, 0);
          ka[(kc + DQ) % (DQ + 1)][1] = kop(kc + DQ, 1);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int mb = 0; mb < kNMB; ++mb)
            s[kb][mb] = mma16(ka[kc % (DQ + 1)][kb], qf[mb][kc], kc == 0 ? negref[mb] : s[kb][mb]);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    auto vop = [&](const bf16* vt, int half, int db) {
      return lds_tr8(vt, F::LSV, half * 32 + lg * 4, half * 32 + 16 + lg * 4, db * 16);
    };
    auto values_ahead = [&](const bf16* vt, int half, const v8 (&pb)[kNMB]) {
      constexpr int DV = DR > 32 ? (CAUSAL ? 1 : 2) : 3;  // (the masked variant's limited body keeps more live)
      v8 va[DV + 1];
#pragma unroll
      for (int d = 0; d < DV; ++d)
        if (d < F::NDB) va[d] = vop(vt, half, d);
#pragma unroll
      for (int db = 0; db < F::NDB; ++db) {
        if (db + DV < F::NDB) va[(db + DV) % (DV + 1)] = vop(vt, half, db + DV);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mb = 0; mb < kNMB; ++mb) o[db][mb] = mma16(va[db % (DV + 1)], pb[mb], o[db][mb]);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    auto step = [&](int pos, auto cur_c, auto limited_c) {
      constexpr int CUR = decltype(cur_c)::value;
      const bf16* kt = CUR == 0 ? k0 : k1;
      const bf16* vt = CUR == 0 ? v0 : v1;
      const bf16* rt = CUR == 0 ? r0 : r1;
      if (pos + 1 < n_visit) {
        if constexpr (CUR == 0) issue(pos + 1, k1, v1, r1);
        else issue(pos + 1, k0, v0, r0);
      }
      const int kbase = tile_of(pos) * kBN;
#pragma unroll 1
      for (int half = 0; half < NKC2; ++half) {
        sblk s;
        scores_ahead(kt, rt, half, s);
        v8 pb[kNMB];
        probs(s, pb, kbase + half * 32, limited_c);
        values_ahead(vt, half, pb);
      }
      __builtin_amdgcn_s_waitcnt(0);  // direct loads of the next tile have landed
      __syncthreads();
    };

    if (n_visit > 0) {
      issue(0, k0, v0, r0);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      // reference of each row: the maximum of its scores over the first 32 keys
      const int kbase = tile_of(0) * kBN;
      sblk s;
      const f32x4 zs[kNMB] = {};
      scores(k0, r0, 0, s, zs);
      // (frame-causal: over the visible keys among them, else over all of them)
#pragma unroll
      for (int mb = 0; mb < kNMB; ++mb) {
        float mx = -__builtin_inff(), mx_all = -__builtin_inff();
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = kbase + kb * 16 + lg * 4 + i;
            if (key < n_keys) {
              mx_all = fmaxf(mx_all, s[kb][mb][i]);
              if (key < vis_end(mb)) mx = fmaxf(mx, s[kb][mb][i]);
            }
          }
        mx = wave_max_across_groups(mx);
        if constexpr (CAUSAL) {
          mx_all = wave_max_across_groups(mx_all);
          mx = mx > -__builtin_inff() ? mx : mx_all;
        }
        negref[mb] = f32x4{-mx, -mx, -mx, -mx};
      }
      step(0, B0(), std::true_type());
      int pos = 1;
      if constexpr (CAUSAL) {
        for (; pos + 1 < n_lim; pos += 2) {
          step(pos, B1(), std::true_type());
          step(pos + 1, B0(), std::true_type());
        }
        if (pos < n_lim) step(pos++, B1(), std::true_type());
      }
      for (; pos + 1 < n_visit; pos += 2) {
        step(pos, B1(), std::false_type());
        step(pos + 1, B0(), std::false_type());
      }
      if (pos < n_visit) step(pos, B1(), std::false_type());
    }

    // epilogue: a lane holds four consecutive outputs of one row. A row that
    // sees keys of this segment but whose sum left [2^-100, 2^100] (its
    // reference came from keys it cannot see, or its scores spread beyond
    // the bound) goes to the exact fallback.
    bool sees[kNMB];
#pragma unroll
    for (int mb = 0; mb < kNMB; ++mb) sees[mb] = n_visit > 0 && tile_begin * kBN < vis_end(mb);
    const int eln = opaque_h(lane);
    const int eli = eln & 15, elg = eln >> 4;
#pragma unroll
    for (int mb = 0; mb < kNMB; ++mb) {
      const float l = wave_sum_across_groups(l_run[mb]);
      const int tok = tok_wave + mb * 16 + eli;
      if (tok >= p.Nq) continue;
      const bool ok = l <= kHeadsSumLimit && (l >= kHeadsSumMin || !sees[mb]);  // false for inf / NaN
      const float inv = (ok && l > 0.f) ? 1.f / l : 0.f;
      if (whole) {
        bf16* dst = (bf16*)p.out + (((size_t)b * p.Nq + tok) * p.H + h) * DH;
#pragma unroll
        for (int db = 0; db < F::NDB; ++db)
          store4_bf16(dst + db * 16 + elg * 4, o[db][mb][0] * inv, o[db][mb][1] * inv, o[db][mb][2] * inv,
                      o[db][mb][3] * inv);
        if (!ok && elg == 0) p.fallback_rows[atomicAdd(p.fallback_count, 1)] = bh * p.Nq + tok;
      } else {
        const size_t prow =
            ((size_t)g * 2 + (first_seg ? 0 : 1)) * F::kRowsBlock + (tok - rb * F::kRowsBlock);
        bf16* dst = (bf16*)p.part_o + prow * DH;
#pragma unroll
        for (int db = 0; db < F::NDB; ++db)
          store4_bf16(dst + db * 16 + elg * 4, o[db][mb][0] * inv, o[db][mb][1] * inv, o[db][mb][2] * inv,
                      o[db][mb][3] * inv);
        // log2 of the piece's weight (reference + log2 of the sum; -inf for a
        // piece without keys the row sees) and its status (+inf: exact fallback)
        if (elg == 0) {
          const bool weighted = ok && l > 0.f;
          p.part_l[prow * 2] = weighted ? -negref[mb][0] + __builtin_amdgcn_logf(l) : -__builtin_inff();
          p.part_l[prow * 2 + 1] = ok ? 0.f : __builtin_inff();
        }
      }
    }
  }
}

// Merge of the partial results of a row block shared by work-groups g0..g1
// (the work-groups whose unit ranges meet the row block's units [a, a + nt)):
// piece g holds o_g / l_g and lw_g = r_g + log2 l_g; with M = max_g lw_g and
// w_g = 2^(lw_g - M), out = sum_g w_g (o_g / l_g) / sum_g w_g. Pieces with
// no key the row sees have lw_g = -inf and weigh 0; a flagged piece sends
// the row to the exact fallback. A work-group takes 32 rows of one row block.
constexpr int kHeadsMergeRows = 32;

template <int DH>
__global__ __launch_bounds__(256) void heads_combine_kernel(HeadsParams p) {
  constexpr int RB = kHeadsRowsPerBlock, NCH = DH / 8;
  static_assert(RB % kHeadsMergeRows == 0, "merge groups tile a row block");
  __shared__ long long slot_base[kMaxMergePieces];
  // row blocks from rb_whole on (the ones dealt whole in rounds are done)
  const long long rbg = p.rb_whole + blockIdx.x / (RB / kHeadsMergeRows);
  const int row_lo = (int)(blockIdx.x % (RB / kHeadsMergeRows)) * kHeadsMergeRows;
  long long a;
  int nt;
  row_block_units(p.classes, p.n_rb, rbg, a, nt);
  const long long Gr = p.grid_rest, rest = p.units - p.u_rest;
  // largest g whose range of the remaining units starts at or before unit x
  auto owner = [&](long long x) { return ((x - p.u_rest + 1) * Gr - 1) / rest; };
  const long long g0 = owner(a), g1 = owner(a + nt - 1);
  if (g0 == g1) return;  // one work-group covered the row block and wrote it
  const int np = (int)(g1 - g0 + 1);  // <= kMaxMergePieces by the host's cap on G'
  if ((int)threadIdx.x < np) {
    const long long g = g0 + threadIdx.x;
    const long long start = p.u_rest + g * rest / Gr;
    slot_base[threadIdx.x] = (g * 2 + (start >= a ? 0 : 1)) * RB;
  }
  __syncthreads();
  const int bh = (int)(rbg / p.n_rb), rb = (int)(rbg - (long long)bh * p.n_rb);
  const int h = bh % p.H, b = bh / p.H;
  const int rows = min(kHeadsMergeRows, p.Nq - rb * RB - row_lo);
  for (int e = threadIdx.x; e < rows * NCH; e += blockDim.x) {
    const int local = row_lo + e / NCH, c0 = (e % NCH) * 8;
    float M = -__builtin_inff();
    bool ok = true;
    for (int k = 0; k < np; ++k) {
      const size_t pr = (size_t)slot_base[k] + local;
      M = fmaxf(M, p.part_l[pr * 2]);
      ok = ok && (p.part_l[pr * 2 + 1] <= kHeadsSumLimit);
    }
    float L = 0.f, acc[8] = {};
    if (M > -__builtin_inff()) {
      for (int k = 0; k < np; ++k) {
        const size_t pr = (size_t)slot_base[k] + local;
        const float wl = fast_exp2(p.part_l[pr * 2] - M);
        L += wl;
        float v[8];
        unpack8<bf16>(load8<bf16>((const bf16*)p.part_o + pr * DH + c0), v);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += wl * v[i];
      }
    }
    const float inv = (ok && L > 0.f) ? 1.f / L : 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] *= inv;
    const int tok = rb * RB + local;
    store8<bf16>((bf16*)p.out + (((size_t)b * p.Nq + tok) * p.H + h) * DH + c0, pack8<bf16>(acc));
    if (!ok && c0 == 0) p.fallback_rows[atomicAdd(p.fallback_count, 1)] = bh * p.Nq + tok;
  }
}

// Rows listed by the attention kernel, recomputed with the textbook two-pass
// softmax over the expanded keys and values. One work-group per listed row
// (grid-stride over the list).
template <int DH, int DR, bool CAUSAL>
__global__ __launch_bounds__(256) void heads_exact_kernel(HeadsParams p) {
  constexpr int QP = DH + DR, CHUNK = 256;
  __shared__ float q[QP];
  __shared__ float pr[CHUNK];
  __shared__ float red[256];
  __shared__ int n_valid_sh;
  __shared__ int frame_of[kSlots];
  const int tid = threadIdx.x;
  const int count = *p.fallback_count;
  for (int idx = blockIdx.x; idx < count; idx += gridDim.x) {
    const int row = p.fallback_rows[idx];  // (b * H + h) * Nq + i
    const int bh = row / p.Nq, i = row - bh * p.Nq, h = bh % p.H, b = bh / p.H;
    __syncthreads();
    if (tid < 64) {
      const int f = tid < p.W ? p.slot_frame[b * p.W + tid] : -1;
      const int rank = window_rank(f, tid);
      if (f >= 0) frame_of[rank] = f;
      const unsigned long long mask = __ballot(f >= 0);
      if (tid == 0) n_valid_sh = __popcll(mask);
    }
    for (int d = tid; d < QP; d += 256) q[d] = to_f<bf16>(((const bf16*)p.q_cat)[(size_t)row * QP + d]);
    __syncthreads();
    const int n_keys = n_valid_sh * p.T;
    // frame-causal variant: keys of frames after the row's query frame are skipped
    const int qframe = p.q_frame_first + i / p.T;
    auto visible = [&](int v) { return !CAUSAL || frame_of[v / p.T] <= qframe; };
    const size_t head_rows = (size_t)bh * p.W * p.T;
    const bf16* kx = (const bf16*)p.k_exp + head_rows * DH;
    const bf16* vx = (const bf16*)p.v_exp + head_rows * DH;
    const bf16* kr = (const bf16*)p.krot + (size_t)b * p.W * p.T * DR;
    auto score = [&](int v) {
      float s = 0.f;
      for (int d = 0; d < DH; ++d) s += q[d] * to_f<bf16>(kx[(size_t)v * DH + d]);
      for (int d = 0; d < DR; ++d) s += q[DH + d] * to_f<bf16>(kr[(size_t)v * DR + d]);
      return s;
    };
    float mx = -__builtin_inff();
    for (int v = tid; v < n_keys; v += 256)
      if (visible(v)) mx = fmaxf(mx, score(v));
    red[tid] = mx;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
      if (tid < s) red[tid] = fmaxf(red[tid], red[tid + s]);
      __syncthreads();
    }
    const float m = red[0];
    __syncthreads();
    float acc = 0.f, lsum = 0.f;
    for (int j0 = 0; j0 < n_keys; j0 += CHUNK) {
      const int v = j0 + tid;
      pr[tid] = v < n_keys && visible(v) ? fast_exp2(score(v) - m) : 0.f;  // scores are log2-scaled
      __syncthreads();
      if (tid < DH) {
        const int nv = min(CHUNK, n_keys - j0);
        for (int j = 0; j < nv; ++j) {
          acc += pr[j] * to_f<bf16>(vx[(size_t)(j0 + j) * DH + tid]);
          lsum += pr[j];
        }
      }
      __syncthreads();
    }
    if (tid < DH)
      ((bf16*)p.out)[(((size_t)b * p.Nq + i) * p.H + h) * DH + tid] = (bf16)(n_keys > 0 && lsum > 0.f ? acc / lsum : 0.f);
  }
}

template <int DC, int DR, int DH, bool CAUSAL>
static hipError_t launch_heads_t(const HeadsParams& p, bool split, hipStream_t s) {
  typedef HeadsTile<DH, DR> F;
  const int nk_max = p.W * p.T;
  hipLaunchKernelGGL((expand_kv_kernel<DC, DR, DH>), dim3((nk_max + kExpKeys - 1) / kExpKeys, p.H, p.batch),
                     dim3(512), 0, s, p);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const long long pieces = (long long)p.batch * p.Nq * p.H * ((DH + DR) / 8);
  hipLaunchKernelGGL((heads_qcat_kernel<DH, DR>), dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, s, p);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL((heads_flash_kernel<DH, DR, CAUSAL>), dim3(p.grid), dim3(F::kThreads), 0, s, p);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (split && (long long)p.batch * p.H * p.n_rb > p.rb_whole) {
    hipLaunchKernelGGL((heads_combine_kernel<DH>),
                       dim3(((long long)p.batch * p.H * p.n_rb - p.rb_whole) * (kHeadsRowsPerBlock / kHeadsMergeRows)),
                       dim3(256), 0, s, p);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  hipLaunchKernelGGL((heads_exact_kernel<DH, DR, CAUSAL>), dim3(kFallbackBlocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

bool heads_supported(int dtype, int d_c, int d_rope, int d_head) {
  return dtype == 0 && d_head == 128 &&
         ((d_c == 192 && d_rope == 32) || (d_c == 128 && d_rope == 32) || (d_c == 160 && d_rope == 64) ||
          (d_c == 192 && d_rope == 64));
}

int heads_tile_keys(int d_head, int d_rope) {
  if (d_head != 128) return 0;
  if (d_rope == 32) return HeadsTile<128, 32>::kBN;
  if (d_rope == 64) return HeadsTile<128, 64>::kBN;
  return 0;
}

template <int DC, int DR>
static hipError_t launch_heads_c(const HeadsParams& p, bool split, bool causal, hipStream_t s) {
  return causal ? launch_heads_t<DC, DR, 128, true>(p, split, s) : launch_heads_t<DC, DR, 128, false>(p, split, s);
}

hipError_t launch_heads(int d_c, int d_rope, int d_head, const HeadsParams& p, bool split, bool causal,
                        hipStream_t s) {
  if (p.batch <= 0 || p.Nq <= 0 || p.grid <= 0) return hipSuccess;
  if (d_head != 128) return hipErrorInvalidValue;
  if (d_c == 192 && d_rope == 32) return launch_heads_c<192, 32>(p, split, causal, s);
  if (d_c == 128 && d_rope == 32) return launch_heads_c<128, 32>(p, split, causal, s);
  if (d_c == 160 && d_rope == 64) return launch_heads_c<160, 64>(p, split, causal, s);
  if (d_c == 192 && d_rope == 64) return launch_heads_c<192, 64>(p, split, causal, s);
  return hipErrorInvalidValue;
}

}  // namespace mla
