// Latent flash attention: the core of one VideoMLA chunk step.
//
// hyper.ai summary of VideoMLA, Method section: head h scores key j with
// q_nope . (W_uk[h] c_j) + q_rope . R(p_j) kR_j and takes the value
// W_uv[h] c_j, so one read of the cached [c_j | kR_j] serves every head.
// chatpaper.ai abstract: the keys are the frames of a fixed-size sliding
// window. With the absorbed query (already multiplied by c = scale * log2 e)
// q_abs = c [W_uk[h]^T q_nope | R(p_i) qR | 0] this file computes, for every
// row (b, i, h),
//   s_j   = q_abs . [c_j | R(t_j, y_j, x_j) kR_j | 0]      (log2 units)
//   o_lat = sum_j 2^(s_j) c_j / sum_j 2^(s_j)
// over every key of every valid ring slot.
//
// Softmax with a fixed per-row reference. 2^s is shift-invariant, so any
// reference r_i gives the same o. Each row takes r_i = the exact maximum of
// its scores over the first 32 keys it visits; later keys may score higher,
// so a probability can exceed 1, but fp32 (and bf16) reach 2^127 and the
// largest probability is at least 1, so nothing underflows. The reference is
// folded into the score product itself (the first product of every score
// block starts from -r_i instead of 0), so a probability costs one exp2; no
// running maximum is tracked and the output accumulators are never rescaled.
// A row whose probability sum exceeds 2^100 (a logit gap beyond ~70 nats) is
// listed and recomputed by an exact two-pass kernel.
//
// Layout of the work (bf16):
//   * the 12 heads of a query are consecutive rows (all heads share the
//     keys); a work-group owns 256 rows in 8 waves of 32 rows (two 16-row
//     blocks), two waves per SIMD, so one wave's exp2 work overlaps the
//     other's matrix products; queries stay in registers for the key loop;
//   * keys stream in 64-key tiles through LDS, double-buffered, one barrier
//     per tile. The latent part goes global -> LDS directly (no registers);
//     the kR part goes through registers and is rotated by 3D-RoPE on its way
//     into LDS. LDS rows are 480 bytes apart, which keeps both LDS read
//     patterns below free of bank conflicts;
//   * scores are formed transposed, S^T = K Q^T (keys as rows), so a lane
//     holds 4 keys of one query row and the probabilities already sit in the
//     lane layout of the B operand of O^T = C^T P^T. The C^T operand is read
//     from the same LDS tile with the transposing LDS load: the latent is
//     staged once for both products;
//   * kv_splits > 1 partitions the key tiles; each split keeps its own
//     reference and a second pass merges the (reference, output, sum) triples.
#include <type_traits>

#include "mla_common.hpp"
#include "mla_internal.hpp"
#include "rope_device.hpp"

namespace mla {

namespace {
constexpr int kMaxSlots = 64;
constexpr float kSumLimit = 1.2676506e30f;  // 2^100
}  // namespace

// bf16: 8 waves x 32 rows (two waves per SIMD) and 64-key tiles; float
// operands are twice as wide, so float runs 4 waves x 32 rows with 32-key
// tiles (it exists for the fp32 configurations, where precision rather than
// speed is the point).
template <typename T, int DC, int DR>
struct FlashTile {
  static constexpr bool kBf16 = sizeof(T) == 2;
  static constexpr int kWaves = kBf16 ? 8 : 4;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kBN = kBf16 ? 64 : 32;           // keys per tile
  static constexpr int kNMB = 2;                        // 16-row blocks per wave
  static constexpr int kRowsWave = kNMB * 16;
  static constexpr int kRowsBlock = kWaves * kRowsWave;
  static constexpr int NKC2 = kBN / 32;                 // 32-key halves per tile
  static constexpr int KP = (DC + DR + 31) / 32 * 32;   // contraction width of QK (zero padded)
  static constexpr int DK = DC + DR;                    // cached row width
  static constexpr int NKC = KP / 32;
  static constexpr int NDB = DC / 16;
  static constexpr int CB = 16 / sizeof(T);             // elements per 16-byte chunk
  static constexpr int LS = kBf16 ? KP + 16 : KP + CB;  // LDS row stride (elements)
  static constexpr int CPR = LS / CB;                   // 16-byte chunks per LDS row
  static constexpr int CC = DC / CB;                    // latent chunks per key
  static constexpr int RC = DR / CB;                    // kR chunks per key
  static constexpr int PADC = (KP - DK) / CB;           // zero chunks read by QK
  static constexpr int TILE_CHUNKS = kBN * CPR;
  static constexpr int N_INSTR = (TILE_CHUNKS + 63) / 64;  // direct-load instructions per tile
  static constexpr int N_INSTR_WAVE = (N_INSTR + kWaves - 1) / kWaves;
  static constexpr int TILE_ELEMS = N_INSTR * 64 * CB;  // LDS elements per buffer (whole instructions)
  static constexpr int RU = 4;                          // kR elements rotated per thread (two pairs)
  static constexpr int NU = DR / RU;                    // rotation units per key
  static constexpr int RCH = kBN * NU;                  // rotation units per tile
  static_assert(DR % RU == 0 && RCH <= kThreads, "one rotation unit per thread");
  static_assert(LS % 4 == 0 && (LS * sizeof(T)) % 16 == 0, "LDS rows must stay 16-byte aligned");
};

// Clears the count of rows handed to the exact fallback.
__global__ void flash_prep_kernel(FlashParams p) { *p.fallback_count = 0; }

// ---------------------------------------------------------------- main kernel
template <typename T, int DC, int DR>
__global__ __launch_bounds__((FlashTile<T, DC, DR>::kThreads), 1) void flash_mla_kernel(FlashParams p) {
  typedef FlashTile<T, DC, DR> F;
  typedef typename V8<T>::type v8;
  constexpr int kBN = F::kBN, kNMB = F::kNMB, kWaves = F::kWaves;
  // Two separately declared buffers (not one 2-D array): with the parity of
  // every access known at compile time, the compiler can tell that reads of
  // one buffer do not depend on the direct global->LDS loads into the other,
  // and does not wait for the prefetch before consuming the current tile.
  __shared__ __attribute__((aligned(16))) T kv0[F::TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) T kv1[F::TILE_ELEMS];
  __shared__ int slot_of[kMaxSlots];
  __shared__ int frame_of[kMaxSlots];
  __shared__ int n_valid_sh;
  __shared__ int4 keytab[2][kBN];     // per key of a tile: {row offset, slot rank, y, x}
  __shared__ f32x2 rcs[kRopeLdsEntries];  // (cos, sin): t rows by slot rank, then y rows, then x rows

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int b = blockIdx.z, split = blockIdx.y;
  const int row_wave = blockIdx.x * F::kRowsBlock + wave * F::kRowsWave;

  // valid ring slots of stream b in slot order
  if (wave == 0) {
    const int f = lane < p.W ? p.slot_frame[b * p.W + lane] : -1;
    const unsigned long long mask = __ballot(f >= 0);
    if (f >= 0) {
      const int rank = __popcll(mask & ((1ull << lane) - 1ull));
      slot_of[rank] = lane;
      frame_of[rank] = f;
    }
    if (lane == 0) n_valid_sh = __popcll(mask);
  }
  __syncthreads();

  // (cos, sin) of every rotary pair the window's keys need, from the global
  // tables: t by slot rank (frames clamped into the table range), y, x
  const int pt = p.rl.d_t / 2, py = p.rl.d_y / 2, px = p.rl.d_x / 2;
  const int y_base = n_valid_sh * pt, x_base = y_base + p.grid_y * py;
  for (int e = tid; e < x_base + p.grid_x * px; e += F::kThreads) {
    int oc, os;
    if (e < y_base) {
      const int r = e / pt, j = e - r * pt;
      int tt = frame_of[r] - p.rl.t_first;
      tt = tt < 0 ? 0 : (tt >= p.rl.n_t ? p.rl.n_t - 1 : tt);
      oc = p.rl.off_ct + tt * pt + j;
      os = p.rl.off_st + tt * pt + j;
    } else if (e < x_base) {
      oc = p.rl.off_cy + e - y_base;
      os = p.rl.off_sy + e - y_base;
    } else {
      oc = p.rl.off_cx + e - x_base;
      os = p.rl.off_sx + e - x_base;
    }
    rcs[e] = f32x2{p.tables[oc], p.tables[os]};
  }

  const int n_keys = n_valid_sh * p.T;
  const int n_tiles = (n_keys + kBN - 1) / kBN;
  const int tiles_per_split = (n_tiles + p.splits - 1) / p.splits;
  const int tile_begin = split * tiles_per_split;
  const int tile_end = min(n_tiles, tile_begin + tiles_per_split);
  const int n_visit = max(0, tile_end - tile_begin);

  // queries of this wave (B operand of S^T = K Q^T), kept in registers
  v8 qf[kNMB][F::NKC];
  {
    const T* qb = (const T*)p.q_abs + (size_t)b * p.Mb * F::KP;
#pragma unroll
    for (int mb = 0; mb < kNMB; ++mb) {
      const int row = row_wave + mb * 16 + li;
#pragma unroll
      for (int kc = 0; kc < F::NKC; ++kc)
        qf[mb][kc] = row < p.Mb ? load8<T>(qb + (size_t)row * F::KP + kc * 32 + lg * 8) : zero8<T>();
    }
  }
  f32x4 negref[kNMB];  // -reference of this lane's row, in every element
  f32x4 o[F::NDB][kNMB];
  float l_run[kNMB];   // this lane's share of the row's probability sum
#pragma unroll
  for (int mb = 0; mb < kNMB; ++mb) {
    negref[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    l_run[mb] = 0.f;
#pragma unroll
    for (int db = 0; db < F::NDB; ++db) o[db][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const T* cache_b = (const T*)p.cache + (size_t)b * p.W * p.T * F::DK;

  // Per-tile key descriptors {row offset, slot rank, y, x}, written one tile
  // ahead by wave 0 into a ping-pong table, so the address of every load
  // below is one LDS read plus an add. Keys past the end of the window alias
  // the last key (their probabilities are forced to 0). Quotients come from a
  // float reciprocal, exact after one correction for indices below 2^22.
  auto div_floor = [](int a, int d, float inv_d) {
    int q = (int)((float)a * inv_d);
    const int r = a - q * d;
    return q + (r >= d ? 1 : 0) - (r < 0 ? 1 : 0);
  };
  auto describe = [&](int pos, int4* tab) {
    if (wave == 0) {
      const int tile = pos == 0 ? tile_end - 1 : tile_begin + pos - 1;
      const int v = min(tile * kBN + lane, n_keys - 1);
      const int rank = div_floor(v, p.T, p.inv_T), tok = v - rank * p.T;
      const int y = div_floor(tok, p.grid_x, p.inv_grid_x);
      if (lane < kBN) tab[lane] = int4{(slot_of[rank] * p.T + tok) * F::DK, rank, y, tok - y * p.grid_x};
    }
  };

  // ---- latent part: global -> LDS, lane order = LDS order (no registers).
  // Instruction k of this wave covers LDS chunks [64 i, 64 i + 64), i = wave + kWaves k;
  // the key and chunk of each lane's slot do not depend on the tile.
  int lat_key[F::N_INSTR_WAVE];
  int lat_off[F::N_INSTR_WAVE];  // element offset inside the key row, -1 = not a latent chunk
#pragma unroll
  for (int k = 0; k < F::N_INSTR_WAVE; ++k) {
    const int instr = wave + kWaves * k;
    const int pos = instr * 64 + lane;
    const int n = pos / F::CPR, c = pos % F::CPR;
    const bool ok = instr < F::N_INSTR && n < kBN && c < F::CC;
    lat_key[k] = ok ? n : 0;
    lat_off[k] = ok ? c * F::CB : -1;
  }
  auto issue_latent = [&](const int4* tab, T* buf) {
    int ro[F::N_INSTR_WAVE];
#pragma unroll
    for (int k = 0; k < F::N_INSTR_WAVE; ++k) ro[k] = tab[lat_key[k]].x;
#pragma unroll
    for (int k = 0; k < F::N_INSTR_WAVE; ++k) {
      const int instr = wave + kWaves * k;
      if (instr < F::N_INSTR && lat_off[k] >= 0) {
        const T* src = cache_b + ro[k] + lat_off[k];
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                         (MLA_LDS void*)(MLA_LDS T*)(buf + instr * 64 * F::CB), 16, 0, 0);
      }
    }
  };

  // ---- kR part: two rotary pairs per thread via registers, rotated with the
  // LDS (cos, sin) rows on their way into LDS
  typedef typename std::conditional<sizeof(T) == 2, u32x2, u32x4>::type ru_t;  // RU elements
  const bool has_r = tid < F::RCH;
  const int r_key = tid / F::NU, r_unit = tid % F::NU;
  ru_t st_r = {};
  auto fetch_rope = [&](const int4* tab) {
    if (has_r) st_r = *reinterpret_cast<const ru_t*>(cache_b + tab[r_key].x + DC + r_unit * F::RU);
  };
  auto stash_rope = [&](const int4* tab, T* buf) {
    if (has_r) {
      const int4 d = tab[r_key];
      float f[F::RU];
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          f[2 * k] = __uint_as_float(st_r[k] << 16);
          f[2 * k + 1] = __uint_as_float(st_r[k] & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) f[k] = __uint_as_float(st_r[k]);
      }
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int pr = r_unit * 2 + k;
        const int idx = pr < pt ? d.y * pt + pr
                                : (pr < pt + py ? y_base + d.z * py + pr - pt : x_base + d.w * px + pr - pt - py);
        const f32x2 cs = rcs[idx];
        rotate_pair(f[2 * k], f[2 * k + 1], cs.x, cs.y);
      }
      ru_t out;
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const uint32_t lo = __builtin_bit_cast(uint16_t, (bf16)f[2 * k]);
          const uint32_t hi = __builtin_bit_cast(uint16_t, (bf16)f[2 * k + 1]);
          out[k] = lo | (hi << 16);
        }
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) out[k] = __float_as_uint(f[k]);
      }
      *reinterpret_cast<ru_t*>(buf + r_key * F::LS + DC + r_unit * F::RU) = out;
    }
  };

  // zero the padding chunks of both buffers once (they are never written again)
  if constexpr (F::PADC > 0) {
    for (int e = tid; e < 2 * kBN * F::PADC; e += F::kThreads) {
      const int buf = e / (kBN * F::PADC), q = e % (kBN * F::PADC);
      const u32x4 z = {};
      *reinterpret_cast<u32x4*>(&(buf ? kv1 : kv0)[((q / F::PADC) * F::CPR + F::CC + F::RC + q % F::PADC) * F::CB]) = z;
    }
  }

  // ---- one 32-key half of a tile; RAGGED: keys at or past n_keys get
  // probability 0 (only the last tile of the window can be ragged)
  auto half_step = [&](const T* kt, int half, int kbase, auto ragged_c) {
    constexpr bool RAGGED = decltype(ragged_c)::value;
    f32x4 s[2][kNMB];
#pragma unroll
    for (int kc = 0; kc < F::NKC; ++kc) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const v8 a = lds_load8<T>(kt + ((half * 2 + kb) * 16 + li) * F::LS + kc * 32 + lg * 8);
#pragma unroll
        for (int mb = 0; mb < kNMB; ++mb) s[kb][mb] = mma16(a, qf[mb][kc], kc == 0 ? negref[mb] : s[kb][mb]);
      }
    }
    v8 pb[kNMB];
#pragma unroll
    for (int mb = 0; mb < kNMB; ++mb) {
      float f8[8];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float e = fast_exp2(s[kb][mb][i]);
          if constexpr (RAGGED) e = kbase + (half * 2 + kb) * 16 + lg * 4 + i < n_keys ? e : 0.f;
          f8[kb * 4 + i] = e;
          l_run[mb] += e;
        }
      pb[mb] = pack8<T>(f8);
    }
    // O^T[d][row] += C^T[d][key] P^T[key][row]; key slot j of lane group g
    // is key 4g+j (j < 4) or 16+4g+(j-4) of this half, matching S^T's layout
#pragma unroll
    for (int db = 0; db < F::NDB; ++db) {
      const v8 a = lds_tr8(kt, F::LS, half * 32 + lg * 4, half * 32 + 16 + lg * 4, db * 16);
#pragma unroll
      for (int mb = 0; mb < kNMB; ++mb) o[db][mb] = mma16(a, pb[mb], o[db][mb]);
    }
  };

  // ---- one tile: start the loads of tile+1 (descriptors ready), describe
  // tile+2, consume the tile, stash the kR part of tile+1, wait for its
  // latent loads, barrier. PAR = buffer holding this tile (static).
  auto tile_step = [&](int pos, auto par_c, auto ragged_c) {
    constexpr int PAR = decltype(par_c)::value;
    T* cur_buf = PAR ? kv1 : kv0;
    T* nxt_buf = PAR ? kv0 : kv1;
    const bool has_next = pos + 1 < n_visit;
    if (has_next) {
      issue_latent(keytab[PAR ^ 1], nxt_buf);
      fetch_rope(keytab[PAR ^ 1]);
    }
    if (pos + 2 < n_visit) describe(pos + 2, keytab[PAR]);
    const int kbase = (pos == 0 ? tile_end - 1 : tile_begin + pos - 1) * kBN;
#pragma unroll 1
    for (int half = 0; half < F::NKC2; ++half) half_step(cur_buf, half, kbase, ragged_c);
    if (has_next) stash_rope(keytab[PAR ^ 1], nxt_buf);
    __builtin_amdgcn_s_waitcnt(0);  // latent loads of the next tile have landed
    __syncthreads();
  };

  if (tile_begin < tile_end) {
    describe(0, keytab[0]);
    if (n_visit > 1) describe(1, keytab[1]);
  }
  __syncthreads();
  if (tile_begin < tile_end) {
    issue_latent(keytab[0], kv0);
    fetch_rope(keytab[0]);
    stash_rope(keytab[0], kv0);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // reference: exact maximum of each row's scores over the first 32 keys it
  // visits (the first half of position 0)
  if (tile_begin < tile_end) {
    const T* kt = kv0;
    const int kbase = (tile_end - 1) * kBN;  // position 0 visits the last tile
    f32x4 s[2][kNMB];
#pragma unroll
    for (int kc = 0; kc < F::NKC; ++kc) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const v8 a = lds_load8<T>(kt + (kb * 16 + li) * F::LS + kc * 32 + lg * 8);
#pragma unroll
        for (int mb = 0; mb < kNMB; ++mb)
          s[kb][mb] = mma16(a, qf[mb][kc], kc == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : s[kb][mb]);
      }
    }
#pragma unroll
    for (int mb = 0; mb < kNMB; ++mb) {
      float mx = -__builtin_inff();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (kbase + kb * 16 + lg * 4 + i < n_keys) mx = fmaxf(mx, s[kb][mb][i]);
      mx = wave_max_across_groups(mx);
      negref[mb] = f32x4{-mx, -mx, -mx, -mx};
    }
  }

  // Visit order: the (possibly ragged) last tile of the range first, with
  // masking, then the others in order; the sum is order independent. So
  // position 0 always uses buffer 0 and the masking variant, and the loop
  // body holds one static-parity step per buffer.
  typedef std::integral_constant<int, 0> P0;
  typedef std::integral_constant<int, 1> P1;
  typedef std::integral_constant<bool, false> Full;
  typedef std::integral_constant<bool, true> Ragged;
  if (n_visit > 0) tile_step(0, P0(), Ragged());
  int pos = 1;
  for (; pos + 1 < n_visit; pos += 2) {
    tile_step(pos, P1(), Full());
    tile_step(pos + 1, P0(), Full());
  }
  if (pos < n_visit) tile_step(pos, P1(), Full());

  // ---- epilogue
#pragma unroll
  for (int mb = 0; mb < kNMB; ++mb) {
    const float l = wave_sum_across_groups(l_run[mb]);
    const int row = row_wave + mb * 16 + li;
    if (row >= p.Mb) continue;
    if (p.splits == 1) {
      const bool ok = l <= kSumLimit;  // false for inf / NaN as well
      const float inv = (ok && l > 0.f) ? 1.f / l : 0.f;
      T* dst = (T*)p.o_lat + ((size_t)b * p.Mb + row) * DC;
#pragma unroll
      for (int db = 0; db < F::NDB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[db * 16 + lg * 4 + i] = to_t<T>(o[db][mb][i] * inv);
      if (!ok && lg == 0) p.fallback_rows[atomicAdd(p.fallback_count, 1)] = b * p.Mb + row;
    } else {
      const size_t prow = ((size_t)split * p.batch + b) * p.Mb + row;
      float* dst = p.part_o + prow * DC;
#pragma unroll
      for (int db = 0; db < F::NDB; ++db) *reinterpret_cast<f32x4*>(dst + db * 16 + lg * 4) = o[db][mb];
      if (lg == 0) {
        const bool empty = tile_begin >= tile_end;  // no keys: weight 0 in the merge
        p.part_l[prow * 2] = empty ? -__builtin_inff() : -negref[mb][0];
        p.part_l[prow * 2 + 1] = l;
      }
    }
  }
}

// Merge of the per-split (reference, output, probability sum) of one row:
// with M = max_s r_s and w_s = 2^(r_s - M), o = sum_s w_s o_s / sum_s w_s l_s.
template <typename T, int DC>
__global__ __launch_bounds__(256) void flash_combine_kernel(FlashParams p) {
  constexpr int D4 = DC / 4;
  const long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long n_rows = (long long)p.batch * p.Mb;
  if (e >= n_rows * D4) return;
  const long long r = e / D4;
  const int d = (int)(e % D4) * 4;
  float M = -__builtin_inff();
  bool ok = true;
  for (int sp = 0; sp < p.splits; ++sp) {
    const size_t pr = (size_t)sp * n_rows + r;
    M = fmaxf(M, p.part_l[pr * 2]);
    ok = ok && (p.part_l[pr * 2 + 1] <= kSumLimit);
  }
  float L = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (M > -__builtin_inff()) {
    for (int sp = 0; sp < p.splits; ++sp) {
      const size_t pr = (size_t)sp * n_rows + r;
      const float w = fast_exp2(p.part_l[pr * 2] - M);
      L += w * p.part_l[pr * 2 + 1];
      acc += w * *reinterpret_cast<const f32x4*>(p.part_o + pr * DC + d);
    }
  }
  const float inv = (ok && L > 0.f) ? 1.f / L : 0.f;
  T* dst = (T*)p.o_lat + (size_t)r * DC + d;
#pragma unroll
  for (int i = 0; i < 4; ++i) dst[i] = to_t<T>(acc[i] * inv);
  if (!ok && d == 0) p.fallback_rows[atomicAdd(p.fallback_count, 1)] = (int)r;
}

// ---------------------------------------------------------------- exact fallback
// Rows whose probabilities underflowed against the bound are recomputed with
// the textbook two-pass softmax: exact row maximum first, then the weighted
// sum. One work-group per listed row (grid-stride over the list), keys striped
// over threads. Slow, and only reached for rows whose bound was very loose.
template <typename T, int DC, int DR>
__global__ __launch_bounds__(256) void flash_exact_kernel(FlashParams p) {
  constexpr int DK = DC + DR;
  constexpr int KP = (DC + DR + 31) / 32 * 32;
  constexpr int CHUNK = 256;
  __shared__ float q[DK];
  __shared__ float pr[CHUNK];
  __shared__ float red[256];
  __shared__ int slot_of[kMaxSlots];
  __shared__ int frame_of[kMaxSlots];
  __shared__ int n_valid_sh;
  const int tid = threadIdx.x;
  const int count = *p.fallback_count;
  for (int idx = blockIdx.x; idx < count; idx += gridDim.x) {
    const int grow = p.fallback_rows[idx];
    const int b = grow / p.Mb;
    __syncthreads();
    if (tid < 64) {
      const int f = tid < p.W ? p.slot_frame[b * p.W + tid] : -1;
      const unsigned long long mask = __ballot(f >= 0);
      if (f >= 0) {
        const int rank = __popcll(mask & ((1ull << tid) - 1ull));
        slot_of[rank] = tid;
        frame_of[rank] = f;
      }
      if (tid == 0) n_valid_sh = __popcll(mask);
    }
    for (int d = tid; d < DK; d += 256) q[d] = to_f<T>(((const T*)p.q_abs)[(size_t)grow * KP + d]);
    __syncthreads();
    const int n_keys = n_valid_sh * p.T;
    const T* cache_b = (const T*)p.cache + (size_t)b * p.W * p.T * DK;
    auto score = [&](int v) {
      const int rank = v / p.T, tok = v - rank * p.T;
      const T* row = cache_b + ((size_t)slot_of[rank] * p.T + tok) * DK;
      const int y = tok / p.grid_x, x = tok - y * p.grid_x;
      float s = 0.f;
      for (int d = 0; d < DC; ++d) s += q[d] * to_f<T>(row[d]);
      for (int k = 0; k < DR / 2; ++k) {
        float a0 = to_f<T>(row[DC + 2 * k]), a1 = to_f<T>(row[DC + 2 * k + 1]), cs, sn;
        rope_cos_sin(p.rl, p.tables, k, frame_of[rank], y, x, cs, sn);
        rotate_pair(a0, a1, cs, sn);
        s += q[DC + 2 * k] * to_f<T>(to_t<T>(a0)) + q[DC + 2 * k + 1] * to_f<T>(to_t<T>(a1));
      }
      return s;
    };
    // pass 1: exact maximum
    float mx = -__builtin_inff();
    for (int v = tid; v < n_keys; v += 256) mx = fmaxf(mx, score(v));
    red[tid] = mx;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
      if (tid < s) red[tid] = fmaxf(red[tid], red[tid + s]);
      __syncthreads();
    }
    const float m = red[0];
    __syncthreads();
    // pass 2: probabilities chunk by chunk, threads then sweep the latent dims
    float acc = 0.f, lsum = 0.f;
    for (int v0 = 0; v0 < n_keys; v0 += CHUNK) {
      const int v = v0 + tid;
      pr[tid] = v < n_keys ? fast_exp2(score(v) - m) : 0.f;  // scores are log2-scaled
      __syncthreads();
      if (tid < DC) {
        const int nv = min(CHUNK, n_keys - v0);
        for (int j = 0; j < nv; ++j) {
          const int vv = v0 + j;
          const int rank = vv / p.T, tok = vv - rank * p.T;
          acc += pr[j] * to_f<T>(cache_b[((size_t)slot_of[rank] * p.T + tok) * DK + tid]);
          lsum += pr[j];
        }
      }
      __syncthreads();
    }
    if (tid < DC) {
      ((T*)p.o_lat)[(size_t)grow * DC + tid] = to_t<T>(n_keys > 0 && lsum > 0.f ? acc / lsum : 0.f);
    }
  }
}

template <typename T, int DC, int DR>
static hipError_t launch_flash_t(const FlashParams& p, hipStream_t s) {
  typedef FlashTile<T, DC, DR> F;
  hipLaunchKernelGGL(flash_prep_kernel, dim3(1), dim3(1), 0, s, p);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  dim3 grid((p.Mb + F::kRowsBlock - 1) / F::kRowsBlock, p.splits, p.batch);
  hipLaunchKernelGGL((flash_mla_kernel<T, DC, DR>), grid, dim3(F::kThreads), 0, s, p);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (p.splits > 1) {
    const long long total = (long long)p.batch * p.Mb * (DC / 4);
    const int blocks = (int)((total + 255) / 256);
    hipLaunchKernelGGL((flash_combine_kernel<T, DC>), dim3(blocks), dim3(256), 0, s, p);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  hipLaunchKernelGGL((flash_exact_kernel<T, DC, DR>), dim3(kFallbackBlocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_flash(int dtype, int d_c, int d_rope, const FlashParams& p, hipStream_t s) {
  if (p.Mb <= 0 || p.batch <= 0) return hipSuccess;
  if (d_c == 192 && d_rope == 32)
    return dtype == 0 ? launch_flash_t<bf16, 192, 32>(p, s) : launch_flash_t<float, 192, 32>(p, s);
  if (d_c == 16 && d_rope == 8)
    return dtype == 0 ? launch_flash_t<bf16, 16, 8>(p, s) : launch_flash_t<float, 16, 8>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace mla
