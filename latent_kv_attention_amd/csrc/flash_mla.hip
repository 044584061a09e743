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
// listed and recomputed by an exact two-pass kernel. Under the frame-causal
// mask a row may see none of its first 32 keys; it then takes the maximum of
// those (invisible) scores, its visible probabilities can underflow, and a
// row that sees keys but sums below 2^-100 is listed as well.
//
// Layout of the work (bf16):
//   * the 12 heads of a query are consecutive rows (all heads share the
//     keys); a work-group owns 256 rows in 8 waves of 32 rows (two 16-row
//     blocks), two waves per SIMD, so one wave's exp2 work overlaps the
//     other's matrix products; queries stay in registers for the key loop;
//   * the window's positional keys are rotated by 3D-RoPE once per call
//     (rope_window_kernel, into the workspace, in key order), not once per
//     work-group that visits them: every row block visits every key;
//   * keys stream in 128-key tiles through LDS, double-buffered, one barrier
//     per tile. Both parts go global -> LDS directly (no registers): the
//     latent into rows 416 bytes apart, which keeps both LDS read patterns
//     below nearly free of bank conflicts, the rotated kR into a packed
//     region whose 16-byte units are XOR-swizzled by key for the same reason;
//   * within a tile each wave takes 32-key halves one after the other:
//     score products, exponentials, value products; the operand reads run
//     three products ahead of their use (scheduling barriers keep that
//     order), and the other wave of the SIMD runs its products while this
//     one computes exponentials;
//   * scores are formed transposed, S^T = K Q^T (keys as rows), so a lane
//     holds 4 keys of one query row and the probabilities already sit in the
//     lane layout of the B operand of O^T = C^T P^T. The C^T operand is read
//     from the same LDS tile with the transposing LDS load: the latent is
//     staged once for both products;
//   * kv_splits > 1 partitions the key tiles; each split keeps its own
//     reference and a second pass merges the pieces by log2 of their weight.
#include <type_traits>

#include "mla_common.hpp"
#include "mla_internal.hpp"
#include "rope_device.hpp"

namespace mla {

namespace {
constexpr int kMaxSlots = 64;

// A copy of x that the compiler cannot see through. Per-lane addresses
// derived from it are recomputed where they are used (a few integer
// operations) instead of being hoisted out of the key loop and held in
// registers across it, where they would crowd out the loop's own operands.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Operand reads of the tile body run this many products ahead: score
// operands kDQ contraction steps, value operands kDV d-blocks. The two waves
// of a SIMD hide each other's exponentials; what stalls the matrix core is
// the latency of the LDS reads, and the registers left beside the queries
// and output accumulators hold three steps of operands.
constexpr int kDQ = 3, kDV = 3;
constexpr float kSumLimit = 0x1p100f;
constexpr float kSumMin = 0x1p-100f;

// Fourth word of a raw buffer resource (no format conversion, no swizzle):
// byte offsets past num_records read as zero.
constexpr int kBufferWord3 = 0x00020000;
}  // namespace

// bf16: 8 waves x 32 rows (two waves per SIMD) and 128-key tiles; float
// operands are twice as wide, so float runs 4 waves x 32 rows with 32-key
// tiles (it exists for the fp32 configurations, where precision rather than
// speed is the point).
template <typename T, int DC, int DR>
struct FlashTile {
  static constexpr bool kBf16 = sizeof(T) == 2;
  static constexpr int kWaves = kBf16 ? 8 : 4;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kBN = kBf16 ? 128 : 32;          // keys per tile
  static constexpr int kNMB = 2;                        // 16-row blocks per wave
  static constexpr int kRowsWave = kNMB * 16;
  static constexpr int kRowsBlock = kWaves * kRowsWave;
  static constexpr int NKC2 = kBN / 32;                 // 32-key halves per tile
  static constexpr int KP = (DC + DR + 31) / 32 * 32;   // contraction width of QK (zero padded)
  static constexpr int DK = DC + DR;                    // cached row width
  static constexpr int NKC = KP / 32;
  static constexpr int NDB = DC / 16;
  static constexpr int CB = 16 / sizeof(T);             // elements per 16-byte chunk
  // Latent region of a tile buffer: one row of LS elements per key, the d_c
  // latent values then 32 bytes of padding for bf16 (a 416-byte stride at
  // d_c = 192, which keeps both operand read patterns nearly free of bank
  // conflicts).
  static constexpr int LS = kBf16 ? DC + 16 : KP + CB;  // LDS row stride (elements)
  static constexpr int CPR = LS / CB;                   // 16-byte chunks per LDS row
  static constexpr int CC = DC / CB;                    // latent chunks per key
  static constexpr int TILE_CHUNKS = kBN * CPR;
  static constexpr int N_INSTR = (TILE_CHUNKS + 63) / 64;  // direct-load instructions per tile
  static constexpr int N_INSTR_WAVE = (N_INSTR + kWaves - 1) / kWaves;
  static constexpr int TILE_ELEMS = N_INSTR * 64 * CB;  // LDS elements per buffer (whole instructions)
  // Rotated-kR region: DR elements per key, no padding, in units of 8
  // elements (the S^T read granularity) whose order within a key is
  // XOR-swizzled by the key index.
  static constexpr int U8 = DR / 8;                     // 8-element units per key
  static constexpr int CPU = 8 * (int)sizeof(T) / 16;   // 16-byte chunks per unit
  static constexpr int RCK = U8 * CPU;                  // 16-byte chunks per key
  static constexpr int KR_ELEMS = kBN * DR;
  static constexpr int KR_INSTR = (kBN * RCK + 63) / 64;
  static constexpr int KR_INSTR_WAVE = (KR_INSTR + kWaves - 1) / kWaves;
  // unit slot of unit u of tile key n (an involution in u), chosen by
  // measuring the bank conflicts of the S^T reads (16 keys, one unit each)
  // per layout: with 64-byte bf16 keys (4 units) keys 8 apart take
  // disjoint unit pairs (conflict-free; XOR by (n / 4) mod 4 conflicted
  // 2-way), with 128-byte keys XOR by (n / 2) mod 8 is conflict-free
  static constexpr int KR_SH = U8 >= 16 ? 0 : U8 == 8 ? 1 : U8 == 4 ? 2 : U8 == 2 ? 3 : 4;  // log2(16 / U8)
  __host__ __device__ static constexpr int kr_slot(int n, int u) {
    return sizeof(T) == 2 && U8 == 4 ? (u ^ (((n >> 3) & 1) * 2))
                                     : U8 > 1 && U8 <= 16 ? (u ^ ((n >> KR_SH) & (U8 - 1))) : u;
  }
  static_assert(DC % 16 == 0 && DR % 8 == 0 && (DR / 8 & (DR / 8 - 1)) == 0,
                "latent in 16-wide blocks; kR in a power-of-two number of 8-element units");
  static_assert(LS % 4 == 0 && (LS * sizeof(T)) % 16 == 0, "LDS rows must stay 16-byte aligned");
};

// 3D-RoPE of the window's positional keys, once per call: key v = (slot
// rank r, token tok) of stream b gets R(t, y, x) kR, with t the frame held
// by the slot of rank r (valid slots ranked by frame, window_rank) and
// (y, x) the token's grid cell, rounded to the cache's element type. Row v
// of the stream's block of p.krot. One thread per 8 elements (4 rotary
// pairs, one 16-byte piece in bf16); grid (unit blocks, slots, stream
// groups). Wave 0 of a work-group ranks the slot and sets up the temporal
// angles of its frame: the table's entries where the table covers the frame
// (the table kernel formed them with the same function), else formed here
// (any frame index; the caller's tables only need to cover the query
// frames). The spatial angles come from the tables. It also clears the count
// of rows handed to the exact fallback.
template <typename T, int DC, int DR>
__global__ __launch_bounds__(256) void rope_window_kernel(FlashParams p) {
  constexpr int NP = DR / 2, U = DR / 8;  // rotary pairs, 8-element units per key
  __shared__ float t_cs[2][NP];            // cos, sin of the temporal pairs at the slot's frame
  __shared__ int rank_sh;                  // the slot's rank among the valid slots
  if ((blockIdx.x | blockIdx.y | blockIdx.z | threadIdx.x) == 0) *p.fallback_count = 0;
  const int slot = blockIdx.y;
  const int e = blockIdx.x * 256 + threadIdx.x;
  const bool active = e < p.T * U;
  const int tok = e / U, q = e - tok * U;  // unit q: pairs 4 q .. 4 q + 3
  const int y = tok / p.grid_x, x = tok - y * p.grid_x;
  const int n_tp = p.rl.d_t / 2;
  for (int b = blockIdx.z; b < p.batch; b += gridDim.z) {
    const int32_t* sf = p.slot_frame + (size_t)b * p.W;
    // this unit's kR values and spatial angles, requested before the slot's
    // rank and temporal angles (neither depends on them)
    float a[8];
    float cs[4], sn[4];
    if (active) {
      unpack8<T>(load8<T>((const T*)p.cache + (((size_t)b * p.W + slot) * p.T + tok) * (DC + DR) + DC + 8 * q), a);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (4 * q + j >= n_tp) rope_cos_sin(p.rl, p.tables, 4 * q + j, 0, y, x, cs[j], sn[j]);
    }
    const int f = sf[slot];  // uniform over the work-group
    if (f < 0) continue;
    __syncthreads();  // the previous stream's rank and angles are no longer read
    if (threadIdx.x < 64) {
      const int lane = threadIdx.x;
      const int r = window_rank(lane < p.W ? sf[lane] : -1, lane);
      if (lane == slot) rank_sh = r;
      if (lane < n_tp) {
        if (f >= p.rl.t_first && f < p.rl.t_first + p.rl.n_t) {
          const int off = (f - p.rl.t_first) * n_tp + lane;
          t_cs[0][lane] = p.tables[p.rl.off_ct + off];
          t_cs[1][lane] = p.tables[p.rl.off_st + off];
        } else {
          rope_axis_cos_sin(p.rope_base, f, lane, p.rl.d_t, &t_cs[0][lane], &t_cs[1][lane]);
        }
      }
    }
    __syncthreads();
    if (!active) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = 4 * q + j;
      if (k < n_tp) {
        cs[j] = t_cs[0][k];
        sn[j] = t_cs[1][k];
      }
      rotate_pair(a[2 * j], a[2 * j + 1], cs[j], sn[j]);
    }
    T* dst = (T*)p.krot + ((size_t)b * p.W * p.T + (size_t)rank_sh * p.T + tok) * DR + 8 * q;
    store8<T>(dst, pack8<T>(a));
  }
}

// ---------------------------------------------------------------- main kernel
// CAUSAL: the frame-causal variant (a query of frame f attends only keys of
// frames <= f); tiles whose keys are all visible to the row block run
// unmasked, tiles with no visible key are skipped, the rest are masked per
// key.
template <typename T, int DC, int DR, bool CAUSAL>
__global__ __launch_bounds__((FlashTile<T, DC, DR>::kThreads), 1) void flash_mla_kernel(FlashParams p) {
  typedef FlashTile<T, DC, DR> F;
  typedef typename V8<T>::type v8;
  constexpr int kBN = F::kBN, kNMB = F::kNMB, kWaves = F::kWaves, NKC2 = F::NKC2;
  // Two separately declared tile buffers (not one 2-D array). Position p of
  // the key loop uses buffer p mod 2 and the loop is unrolled twice, so every
  // buffer access has a compile-time buffer: the compiler can then tell that
  // reads of the current tile do not depend on the direct global->LDS loads
  // into the other buffer, and does not wait for the prefetch before reading.
  __shared__ __attribute__((aligned(16))) T kv0[F::TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) T kv1[F::TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) T kr0[F::KR_ELEMS];
  __shared__ __attribute__((aligned(16))) T kr1[F::KR_ELEMS];
  __shared__ int slot_of[kMaxSlots];
  __shared__ int frame_of[kMaxSlots];  // frame held by the r-th valid slot (frame-causal variant)
  __shared__ int n_valid_sh;
  __shared__ int keytab[2][kBN];  // per key of a tile: byte offset of its cache row

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;

  // Direct-load slots of this lane: instruction k of the wave fills LDS
  // chunks [64 i, 64 i + 64), i = wave + kWaves k; the lane's chunk is chunk
  // c of key n. Packed as (n << 16) | (byte offset of the chunk in the key
  // row), or -1 where the chunk is not part of the latent.
  int lat_pk[F::N_INSTR_WAVE];
#pragma unroll
  for (int k = 0; k < F::N_INSTR_WAVE; ++k) {
    const int instr = wave + kWaves * k;
    const int pos = instr * 64 + lane;
    const int n = pos / F::CPR, c = pos - n * F::CPR;
    lat_pk[k] = (instr < F::N_INSTR && n < kBN && c < F::CC) ? (n << 16) | (c * 16) : -1;
  }
  // Rotated-kR slots: instruction k of the wave fills chunks [64 i, 64 i + 64)
  // of the kR region, i = wave + kWaves k; the lane's chunk holds unit slot
  // us of key n, i.e. unit kr_slot(n, us) of the key's row in the rotated
  // buffer. Packed as (n << 16) | (byte offset in that row), or -1.
  int kr_pk[F::KR_INSTR_WAVE];
#pragma unroll
  for (int k = 0; k < F::KR_INSTR_WAVE; ++k) {
    const int instr = wave + kWaves * k;
    const int q = instr * 64 + lane;
    const int n = q / F::RCK, cs = q - n * F::RCK;
    const int us = cs / F::CPU, ci = cs - us * F::CPU;
    kr_pk[k] = (instr < F::KR_INSTR && n < kBN) ? (n << 16) | ((F::kr_slot(n, us) * F::CPU + ci) * 16) : -1;
  }

  // Work-group g (logical index) first takes its whole row blocks, one per
  // round (row block k G + g): all work-groups start a round together and
  // walk the keys in the same order, so the work-groups of an XCD, which
  // hold consecutive row blocks, read the same key tiles at the same time
  // and share them through its L2. Then its range of the remaining units,
  // [u_rest + g R / G', u_rest + (g + 1) R / G'), as consecutive segments of
  // at most one row block each. A segment that covers its whole row block
  // writes the normalised output; a partial one writes (output, reference,
  // sum) to slot 0 (the work-group's first segment of the range) or 1 (its
  // last) for the merge pass.
  const long long G = p.grid;
  const int g = xcd_major(blockIdx.x, p.grid);
  const long long rounds = p.rb_whole / G;
  const long long rest = p.units - p.u_rest;
  const long long u_first = g < p.grid_rest ? p.u_rest + (long long)g * rest / p.grid_rest : p.units;
  const long long u_last = g < p.grid_rest ? p.u_rest + ((long long)g + 1) * rest / p.grid_rest : p.units;
  //
  // Segments of the range are taken last to first: a range that ends inside
  // a row block starts with that block's first tiles, so at any moment most
  // work-groups read the same few key tiles and share them through the L2.
  long long round = 0;
  for (long long u = u_last;;) {
    long long rbg, ua;  // row block over all streams, its first unit
    int nt;             // its unit count
    int j0, j1;         // the segment's units within the row block
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
    const int b = (int)(rbg / p.n_rb), rb = (int)(rbg - (long long)b * p.n_rb);
    const int row_wave = rb * F::kRowsBlock + wave * F::kRowsWave;
    __syncthreads();  // LDS of the previous segment is no longer read

    // valid ring slots of stream b in key order (by frame, window_rank)
    if (wave == 0) {
      const int f = lane < p.W ? p.slot_frame[b * p.W + lane] : -1;
      const int rank = window_rank(f, lane);
      if (f >= 0) {
        slot_of[rank] = lane;
        if constexpr (CAUSAL) frame_of[rank] = f;
      }
      const unsigned long long mask = __ballot(f >= 0);
      if (lane == 0) n_valid_sh = __popcll(mask);
    }
    __syncthreads();

    const int n_keys = n_valid_sh * p.T;

    // Frame-causal variant: keys are in frame order, so the keys a row may
    // see are a prefix of the window, those of the valid slots whose frame
    // is at most the row's query frame (rows are (token, head) pairs, H per
    // token, T tokens per frame). vis_end: the end of that prefix for this
    // lane's two rows; vis_lo / n_keys_rb: for the row block's first and
    // last rows (the keys every row sees, and the keys the block visits).
    int vis_end[kNMB];
    int vis_lo = n_keys, n_keys_rb = n_keys;
    if constexpr (CAUSAL) {
      const int rows_per_frame = p.T * p.H;
      auto visible_keys = [&](int qf) {
        int n = 0;
        for (int r = 0; r < n_valid_sh; ++r) n += frame_of[r] <= qf ? 1 : 0;
        return n * p.T;
      };
#pragma unroll
      for (int mb = 0; mb < kNMB; ++mb) {
        const int row = row_wave + mb * 16 + li;
        vis_end[mb] = row < p.Mb ? visible_keys(p.q_frame_first + row / rows_per_frame) : n_keys;
      }
      const int r_first = rb * F::kRowsBlock, r_last = min(r_first + F::kRowsBlock, p.Mb) - 1;
      vis_lo = visible_keys(p.q_frame_first + r_first / rows_per_frame);
      n_keys_rb = visible_keys(p.q_frame_first + r_last / rows_per_frame);
    } else {
#pragma unroll
      for (int mb = 0; mb < kNMB; ++mb) vis_end[mb] = n_keys;
    }
    // this segment's share of the row block's tiles (units map onto the
    // tiles of a full window; a partly filled window scales proportionally)
    const int n_tiles = (n_keys_rb + kBN - 1) / kBN;
    const int tile_begin = (int)((long long)j0 * n_tiles / nt);
    const int tile_end = (int)((long long)j1 * n_tiles / nt);
    const int n_visit = max(0, tile_end - tile_begin);
    // Positions 0 .. n_lim - 1 visit the range's last tiles, last first,
    // through the tile body that gives keys past a limit zero weight (past
    // the window: the last tile can be ragged; frame-causal variant: past
    // the row's visible prefix); the other positions visit the rest of the
    // range in order with the plain body. Frame-causal: the limited tiles
    // are those not seen whole by every row of the block (keys from vis_lo
    // on), at least one, and an odd count where the range allows, so that
    // the plain positions start on the same tile buffer as without the mask.
    int n_lim = n_visit > 0 ? 1 : 0;
    if constexpr (CAUSAL) {
      if (n_visit > 0) {
        int m = max(1, tile_end - max(tile_begin, vis_lo / kBN));
        if (m % 2 == 0) m = min(m + 1, n_visit);
        n_lim = m;
      }
    }

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

    // stream base (uniform); per-key byte offsets fit 32 bits because a window
    // holds at most 2^22 keys of at most 224 elements of at most 4 bytes
    const char* cache_b = (const char*)p.cache + (size_t)b * p.W * p.T * F::DK * sizeof(T);
    // rotated kR of the stream's window, one row of DR elements per key in
    // key order (slot rank major)
    const char* krot_b = (const char*)p.krot + (size_t)b * p.W * p.T * DR * sizeof(T);

    // Per-tile key descriptors (byte offset of the key's cache row), written one
    // tile ahead by wave 0 into a ping-pong table, so the address of
    // every load below is one LDS read plus an add. Keys past the end of the
    // window alias the last key (their scores are masked). Quotients come
    // from a float reciprocal, exact after one correction below 2^22.
    auto div_floor = [](int a, int d, float inv_d) {
      int q = (int)((float)a * inv_d);
      const int r = a - q * d;
      return q + (r >= d ? 1 : 0) - (r < 0 ? 1 : 0);
    };
    auto tile_of = [&](int pos) { return pos < n_lim ? tile_end - 1 - pos : tile_begin + pos - n_lim; };
    auto describe = [&](int pos, int* tab) {
      if (wave < (kBN + 63) / 64) {
        const int ln = opaque(lane) + wave * 64;
        const int v = min(tile_of(pos) * kBN + ln, n_keys - 1);
        const int rank = div_floor(v, p.T, p.inv_T), tok = v - rank * p.T;
        if (ln < kBN) tab[ln] = (slot_of[rank] * p.T + tok) * F::DK * (int)sizeof(T);
      }
    };

    // Buffer resources of the stream's cache and rotated keys. The direct
    // loads use the buffer form: its LDS writes are counted on the vector
    // memory counter alone, so the compiler keeps exact (partial) waits for
    // the LDS operand reads while a tile's loads are in flight.
    const __amdgpu_buffer_rsrc_t cache_rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)cache_b, 0, (int)((size_t)p.W * p.T * F::DK * sizeof(T)), kBufferWord3);
    const __amdgpu_buffer_rsrc_t krot_rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)krot_b, 0, (int)((size_t)p.W * p.T * DR * sizeof(T)), kBufferWord3);
    // ---- latent part: global -> LDS, lane order = LDS order (no registers)
    auto issue_latent = [&](const int* tab, T* buf) {
#pragma unroll
      for (int k = 0; k < F::N_INSTR_WAVE; ++k) {
        const int instr = wave + kWaves * k;
        const int pk = opaque(lat_pk[k]);
        if (instr < F::N_INSTR && pk >= 0) {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(cache_rs, (MLA_LDS void*)(MLA_LDS T*)(buf + instr * 64 * F::CB), 16,
                                                   (unsigned)(tab[pk >> 16] + (pk & 0xffff)), 0, 0, 0);
        }
      }
    };

    // ---- rotated kR part: the tile's keys are consecutive rows of the
    // rotated buffer (keys past the end of the window alias the last key)
    auto issue_rope = [&](int kbase, T* buf) {
#pragma unroll
      for (int k = 0; k < F::KR_INSTR_WAVE; ++k) {
        const int instr = wave + kWaves * k;
        const int pk = opaque(kr_pk[k]);
        if (instr < F::KR_INSTR && pk >= 0) {
          const int v = min(kbase + (pk >> 16), n_keys - 1);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(krot_rs, (MLA_LDS void*)(MLA_LDS T*)(buf + instr * 64 * F::CB), 16,
                                                   (unsigned)(v * DR * (int)sizeof(T) + (pk & 0xffff)), 0, 0, 0);
        }
      }
    };

    // ---- the three pieces of the key loop, for one 32-key half of a tile.
    // Scores S^T = K Q^T of half `half` of the tile in `kt`, seeded with
    // `seed` (the negated reference of each row).
    typedef f32x4 sblk[2][kNMB];
    auto scores = [&](const T* kt, const T* ktr, int half, sblk& s, const f32x4 (&seed)[kNMB]) {
#pragma unroll
      for (int kc = 0; kc < F::NKC; ++kc) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int row = (half * 2 + kb) * 16 + li, dim = kc * 32 + lg * 8;
          auto rope_unit = [&]() {
            return lds_load8<T>(ktr + row * DR + F::kr_slot(row, (dim - DC) / 8) * 8);
          };
          v8 a;
          if ((kc + 1) * 32 <= DC) {
            a = lds_load8<T>(kt + row * F::LS + dim);
          } else if (kc * 32 >= DC && (kc + 1) * 32 <= F::DK) {
            a = rope_unit();
          } else {  // a block mixing latent, kR and zero padding (small shapes)
            a = dim < DC ? lds_load8<T>(kt + row * F::LS + dim) : (dim < F::DK ? rope_unit() : zero8<T>());
          }
#pragma unroll
          for (int mb = 0; mb < kNMB; ++mb) s[kb][mb] = mma16(a, qf[mb][kc], kc == 0 ? seed[mb] : s[kb][mb]);
        }
      }
    };
    auto buf_of = [&](auto par_c) -> T* { return decltype(par_c)::value == 0 ? kv0 : kv1; };
    auto kr_of = [&](auto par_c) -> T* { return decltype(par_c)::value == 0 ? kr0 : kr1; };
    typedef std::integral_constant<int, 0> B0;
    typedef std::integral_constant<int, 1> B1;


    // One tile: start the loads of the next position (descriptors ready),
    // describe the one after, consume this tile half by half, wait for the
    // next tile's loads, barrier.
    auto step = [&](int pos, auto cur_c, auto limited_c) {
      constexpr int CUR = decltype(cur_c)::value;
      typedef std::integral_constant<int, CUR ^ 1> nxt_c;
      T* cur = buf_of(cur_c);
      T* cur_r = kr_of(cur_c);
      const bool has_next = pos + 1 < n_visit;
      if (has_next) {
        issue_latent(keytab[CUR ^ 1], buf_of(nxt_c()));
        issue_rope(tile_of(pos + 1) * kBN, kr_of(nxt_c()));
      }
      if (pos + 2 < n_visit) describe(pos + 2, keytab[CUR]);
      const int kbase = tile_of(pos) * kBN;
      auto halves = [&]() {
        // A operand of the score product S^T = K Q^T: keys 16 kb .. of the
        // half, contraction dims 32 kc .. (latent, rotated kR or zero padding)
        auto kop = [&](int half, int kc, int kb) -> v8 {
          const int row = (half * 2 + kb) * 16 + li, dim = kc * 32 + lg * 8;
          auto rope_unit = [&]() { return lds_load8<T>(cur_r + row * DR + F::kr_slot(row, (dim - DC) / 8) * 8); };
          if ((kc + 1) * 32 <= DC) return lds_load8<T>(cur + row * F::LS + dim);
          if (kc * 32 >= DC && (kc + 1) * 32 <= F::DK) return rope_unit();
          return dim < DC ? lds_load8<T>(cur + row * F::LS + dim) : (dim < F::DK ? rope_unit() : zero8<T>());
        };
        // A operand of the value product O^T[d][row] += C^T[d][key] P^T[key][row]
        // for latent dims 16 db ..: key slot j of lane group lg is key
        // 4 lg + j (j < 4) or 16 + 4 lg + (j - 4) of the half, matching the
        // layout of the scores S^T (so the probabilities never leave registers)
        auto vop = [&](int half, int db) -> v8 {
          return lds_tr8(cur, F::LS, half * 32 + lg * 4, half * 32 + 16 + lg * 4, db * 16);
        };
        constexpr bool LIMITED = decltype(limited_c)::value;
        // exponentials of 16-row block mb, key block kb of a half: 4 values;
        // keys past the window (a ragged tile) and, when masked, keys past
        // the row's visible prefix weigh zero (vis_end <= n_keys)
        auto expo = [&](const sblk& s, float (&f)[kNMB][8], int mb, int kb, int kfirst) {
          // limited body: key kfirst + 4 lg + 16 kb + i is kept when
          // 16 kb + i < lim, the limit being the row's visible prefix under the
          // frame-causal mask (within the window), else the window's end
          int lim = 0;
          if constexpr (LIMITED) lim = (CAUSAL ? vis_end[mb] : n_keys) - kfirst - 4 * opaque(lg);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float e = fast_exp2(s[kb][mb][i]);
            if constexpr (LIMITED) e = kb * 16 + i < lim ? e : 0.f;
            f[mb][kb * 4 + i] = e;
            l_run[mb] += e;
          }
        };
        // one half: the score products (operands read kDQ contraction steps
        // ahead), the exponentials, then the value products (operands read
        // kDV d-blocks ahead); scheduling barriers keep each read that far
        // ahead of its product
        v8 ka[kDQ + 1][2];
        auto fetch = [&](int half, int kc) {
          ka[kc % (kDQ + 1)][0] = kop(half, kc, 0);
          ka[kc % (kDQ + 1)][1] = kop(half, kc, 1);
        };
        auto one_half = [&](int half) {
          sblk s;
#pragma unroll
          for (int d = 0; d < kDQ; ++d)
            if (d < F::NKC) fetch(half, d);
#pragma unroll
          for (int kc = 0; kc < F::NKC; ++kc) {
            if (kc + kDQ < F::NKC) fetch(half, kc + kDQ);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
              for (int mb = 0; mb < kNMB; ++mb)
                s[kb][mb] = mma16(ka[kc % (kDQ + 1)][kb], qf[mb][kc], kc == 0 ? negref[mb] : s[kb][mb]);
            __builtin_amdgcn_sched_barrier(0);
          }
          float f[kNMB][8];
#pragma unroll
          for (int c = 0; c < 2 * kNMB; ++c) expo(s, f, c / 2, c % 2, kbase + half * 32);
          v8 pb[kNMB];
#pragma unroll
          for (int mb = 0; mb < kNMB; ++mb) pb[mb] = pack8<T>(f[mb]);
          v8 va[kDV + 1];
#pragma unroll
          for (int d = 0; d < kDV; ++d)
            if (d < F::NDB) va[d] = vop(half, d);
#pragma unroll
          for (int db = 0; db < F::NDB; ++db) {
            if (db + kDV < F::NDB) va[(db + kDV) % (kDV + 1)] = vop(half, db + kDV);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int mb = 0; mb < kNMB; ++mb) o[db][mb] = mma16(va[db % (kDV + 1)], pb[mb], o[db][mb]);
            __builtin_amdgcn_sched_barrier(0);
          }
        };
#pragma unroll 1
        for (int half = 0; half < NKC2; ++half) one_half(half);
      };
      halves();
      __builtin_amdgcn_s_waitcnt(0);  // direct loads of the next tile have landed
      __syncthreads();
    };

    // ---- prologue: descriptors of positions 0 and 1, tile 0 into buffer 0,
    // then the reference from its first 32 keys
    if (n_visit > 0) {
      describe(0, keytab[0]);
      if (n_visit > 1) describe(1, keytab[1]);
    }
    __syncthreads();
    if (n_visit > 0) {
      issue_latent(keytab[0], kv0);
      issue_rope(tile_of(0) * kBN, kr0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (n_visit > 0) {
      const int kbase = tile_of(0) * kBN;
      sblk s;
      const f32x4 zs[kNMB] = {};
      scores(kv0, kr0, 0, s, zs);
#pragma unroll
      for (int mb = 0; mb < kNMB; ++mb) {
        float mx = -__builtin_inff();
        if constexpr (!CAUSAL) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (kbase + kb * 16 + lg * 4 + i < n_keys) mx = fmaxf(mx, s[kb][mb][i]);
          mx = wave_max_across_groups(mx);
        } else {
          // the maximum over the visible keys among the first 32, else over
          // all of them (a row that sees none of them still gets a reference
          // of the scores' scale)
          float mx_all = -__builtin_inff();
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int key = kbase + kb * 16 + lg * 4 + i;
              if (key < n_keys) {
                mx_all = fmaxf(mx_all, s[kb][mb][i]);
                if (key < vis_end[mb]) mx = fmaxf(mx, s[kb][mb][i]);
              }
            }
          mx = wave_max_across_groups(mx);
          mx_all = wave_max_across_groups(mx_all);
          mx = mx > -__builtin_inff() ? mx : mx_all;
        }
        negref[mb] = f32x4{-mx, -mx, -mx, -mx};
      }
      step(0, B0(), std::true_type());
    }
    {
      int pos = 1;
      if constexpr (CAUSAL) {
        // the other limited positions (n_lim is odd unless it is n_visit)
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

    // ---- epilogue
    // Does row mb see any key of this segment? Every visited key for the
    // unmasked kernel; for the frame-causal one, any key whose frame is at
    // most the row's (skipped tiles hold none: their frames exceed every
    // frame of the row block). A row that sees keys but whose sum stayed
    // below 2^-100 took its reference from keys it cannot see (none of its
    // first 32 visited keys was visible) and may have lost its visible
    // probabilities to underflow; like an overflowing row it goes to the
    // exact fallback.
    bool sees[kNMB];
    if constexpr (CAUSAL) {
      // the segment visits keys from tile_begin kBN on
#pragma unroll
      for (int mb = 0; mb < kNMB; ++mb) sees[mb] = n_visit > 0 && tile_begin * kBN < vis_end[mb];
    } else {
#pragma unroll
      for (int mb = 0; mb < kNMB; ++mb) sees[mb] = n_visit > 0;
    }
    const int eln = opaque(lane);
    const int eli = eln & 15, elg = eln >> 4;
#pragma unroll
    for (int mb = 0; mb < kNMB; ++mb) {
      const float l = wave_sum_across_groups(l_run[mb]);
      const int row = rb * F::kRowsBlock + wave * F::kRowsWave + mb * 16 + eli;
      if (row >= p.Mb) continue;
      // false for inf / NaN as well
      const bool ok = l <= kSumLimit && (l >= kSumMin || !sees[mb]);
      const float inv = (ok && l > 0.f) ? 1.f / l : 0.f;
      if (whole) {
        T* dst = (T*)p.o_lat + ((size_t)b * p.Mb + row) * DC;
#pragma unroll
        for (int db = 0; db < F::NDB; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i) dst[db * 16 + elg * 4 + i] = to_t<T>(o[db][mb][i] * inv);
        if (!ok && elg == 0) p.fallback_rows[atomicAdd(p.fallback_count, 1)] = b * p.Mb + row;
      } else {
        // partial output normalised by its own sum (values of the size of
        // the latent, so the cache's element type holds them), plus, in
        // float for the merge, log2 of the piece's total weight (reference +
        // log2 of the sum; -inf for a piece without keys the row sees) and a
        // status (+inf when the row needs the exact fallback)
        const size_t prow = ((size_t)g * 2 + (first_seg ? 0 : 1)) * F::kRowsBlock + row - rb * F::kRowsBlock;
        T* dst = (T*)p.part_o + prow * DC;
#pragma unroll
        for (int db = 0; db < F::NDB; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i) dst[db * 16 + elg * 4 + i] = to_t<T>(o[db][mb][i] * inv);
        if (elg == 0) {
          const bool weighted = ok && l > 0.f;
          p.part_l[prow * 2] = weighted ? -negref[mb][0] + __builtin_amdgcn_logf(l) : -__builtin_inff();
          p.part_l[prow * 2 + 1] = ok ? 0.f : __builtin_inff();
        }
      }
    }
  }
}

// Merge of the partial results of a row block shared by work-groups
// g0..g1 (the work-groups whose unit ranges meet the row block's units
// [a, a + nt)). Piece g holds o_g / l_g and lw_g = r_g + log2 l_g, the
// log2 of its total weight sum_j 2^(s_j) (r_g its reference); with
// M = max_g lw_g and w_g = 2^(lw_g - M) <= 1 the row is
// o = sum_g w_g (o_g / l_g) / sum_g w_g. The heaviest piece has w_g = 1, so
// a piece can only underflow when its share is below 2^-126; pieces with no
// key the row sees have lw_g = -inf and weigh 0. A piece flagged for the
// exact fallback (status > 2^100) sends the whole row there.
// Work-group g's piece sits in its slot 0 when its range starts inside the
// row block, else in its slot 1. A work-group takes kMergeRows rows of one
// row block: the piece bookkeeping is computed once (uniform), then threads
// sweep (row, 16-byte chunk) pairs.
constexpr int kMergeRows = 32;

template <typename T, int DC, int RB>
__global__ __launch_bounds__(256) void flash_combine_kernel(FlashParams p) {
  constexpr int CH = 16 / sizeof(T);  // values per 16-byte chunk
  constexpr int NCH = DC / CH;
  typedef typename std::conditional<sizeof(T) == 2, u32x4, f32x4>::type chunk_t;
  __shared__ long long slot_base[kMaxMergePieces];  // first partial row of each piece
  // row blocks from rb_whole on (the ones dealt whole in rounds are done)
  const long long rbg = p.rb_whole + blockIdx.x / (RB / kMergeRows);
  const int row_lo = (int)(blockIdx.x % (RB / kMergeRows)) * kMergeRows;
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
  const int b = (int)(rbg / p.n_rb), rb = (int)(rbg - (long long)b * p.n_rb);
  const int rows = min(kMergeRows, p.Mb - rb * RB - row_lo);
  for (int e = threadIdx.x; e < rows * NCH; e += blockDim.x) {
    const int local = row_lo + e / NCH, c0 = (e % NCH) * CH;
    float M = -__builtin_inff();
    bool ok = true;
    for (int k = 0; k < np; ++k) {
      const size_t pr = (size_t)slot_base[k] + local;
      M = fmaxf(M, p.part_l[pr * 2]);
      ok = ok && (p.part_l[pr * 2 + 1] <= kSumLimit);
    }
    float L = 0.f, acc[CH] = {};
    if (M > -__builtin_inff()) {
      for (int k = 0; k < np; ++k) {
        const size_t pr = (size_t)slot_base[k] + local;
        const float wl = fast_exp2(p.part_l[pr * 2] - M);
        L += wl;
        const chunk_t raw = *reinterpret_cast<const chunk_t*>((const T*)p.part_o + pr * DC + c0);
        float v[CH];
        if constexpr (sizeof(T) == 2) {
          unpack8<T>(__builtin_bit_cast(typename V8<T>::type, raw), v);
        } else {
#pragma unroll
          for (int i = 0; i < CH; ++i) v[i] = raw[i];
        }
#pragma unroll
        for (int i = 0; i < CH; ++i) acc[i] += wl * v[i];
      }
    }
    const float inv = (ok && L > 0.f) ? 1.f / L : 0.f;
    const size_t r = (size_t)b * p.Mb + rb * RB + local;
    chunk_t out;
    if constexpr (sizeof(T) == 2) {
      float f[CH];
#pragma unroll
      for (int i = 0; i < CH; ++i) f[i] = acc[i] * inv;
      out = __builtin_bit_cast(chunk_t, pack8<T>(f));
    } else {
#pragma unroll
      for (int i = 0; i < CH; ++i) out[i] = acc[i] * inv;
    }
    *reinterpret_cast<chunk_t*>((T*)p.o_lat + r * DC + c0) = out;
    if (!ok && c0 == 0) p.fallback_rows[atomicAdd(p.fallback_count, 1)] = (int)r;
  }
}

// ---------------------------------------------------------------- exact fallback
// Rows whose probabilities underflowed against the bound are recomputed with
// the textbook two-pass softmax: exact row maximum first, then the weighted
// sum. One work-group per listed row (grid-stride over the list), keys striped
// over threads. Slow, and only reached for rows whose bound was very loose.
template <typename T, int DC, int DR, bool CAUSAL>
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
      const int rank = window_rank(f, tid);
      if (f >= 0) {
        slot_of[rank] = tid;
        frame_of[rank] = f;
      }
      const unsigned long long mask = __ballot(f >= 0);
      if (tid == 0) n_valid_sh = __popcll(mask);
    }
    for (int d = tid; d < DK; d += 256) q[d] = to_f<T>(((const T*)p.q_abs)[(size_t)grow * KP + d]);
    __syncthreads();
    const int n_keys = n_valid_sh * p.T;
    const T* cache_b = (const T*)p.cache + (size_t)b * p.W * p.T * DK;
    // the window's rotated positional keys, as the main kernel read them
    const T* krot_b = (const T*)p.krot + (size_t)b * p.W * p.T * DR;
    // frame-causal variant: keys of frames after the row's query frame are skipped
    const int qframe = p.q_frame_first + (grow - b * p.Mb) / (p.T * p.H);
    auto visible = [&](int v) { return !CAUSAL || frame_of[v / p.T] <= qframe; };
    auto score = [&](int v) {
      const int rank = v / p.T, tok = v - rank * p.T;
      const T* row = cache_b + ((size_t)slot_of[rank] * p.T + tok) * DK;
      const T* kr = krot_b + (size_t)v * DR;
      float s = 0.f;
      for (int d = 0; d < DC; ++d) s += q[d] * to_f<T>(row[d]);
      for (int d = 0; d < DR; ++d) s += q[DC + d] * to_f<T>(kr[d]);
      return s;
    };
    // pass 1: exact maximum
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
    // pass 2: probabilities chunk by chunk, threads then sweep the latent dims
    float acc = 0.f, lsum = 0.f;
    for (int v0 = 0; v0 < n_keys; v0 += CHUNK) {
      const int v = v0 + tid;
      pr[tid] = v < n_keys && visible(v) ? fast_exp2(score(v) - m) : 0.f;  // scores are log2-scaled
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

template <typename T, int DC, int DR, bool CAUSAL>
static hipError_t launch_flash_v(const FlashParams& p, bool split, hipStream_t s) {
  typedef FlashTile<T, DC, DR> F;
  hipLaunchKernelGGL((rope_window_kernel<T, DC, DR>), dim3((p.T * (DR / 8) + 255) / 256, p.W, min(p.batch, 65535)),
                     dim3(256), 0, s, p);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((flash_mla_kernel<T, DC, DR, CAUSAL>), dim3(p.grid), dim3(F::kThreads), 0, s, p);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (split && (long long)p.batch * p.n_rb > p.rb_whole) {
    static_assert(F::kRowsBlock % kMergeRows == 0, "merge groups tile a row block");
    hipLaunchKernelGGL((flash_combine_kernel<T, DC, F::kRowsBlock>),
                       dim3(((long long)p.batch * p.n_rb - p.rb_whole) * (F::kRowsBlock / kMergeRows)), dim3(256), 0,
                       s, p);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  hipLaunchKernelGGL((flash_exact_kernel<T, DC, DR, CAUSAL>), dim3(kFallbackBlocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <typename T, int DC, int DR>
static hipError_t launch_flash_t(const FlashParams& p, bool split, bool causal, hipStream_t s) {
  return causal ? launch_flash_v<T, DC, DR, true>(p, split, s) : launch_flash_v<T, DC, DR, false>(p, split, s);
}

template <typename T, int DC, int DR>
static hipError_t launch_rope_window_t(const FlashParams& p, hipStream_t s) {
  hipLaunchKernelGGL((rope_window_kernel<T, DC, DR>), dim3((p.T * (DR / 8) + 255) / 256, p.W, min(p.batch, 65535)),
                     dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_rope_window(int dtype, int d_c, int d_rope, const FlashParams& p, hipStream_t s) {
  if (p.batch <= 0) return hipSuccess;
#define MLA_ROPE_CASE(DCV, DRV) \
  if (d_c == DCV && d_rope == DRV) \
    return dtype == 0 ? launch_rope_window_t<bf16, DCV, DRV>(p, s) : launch_rope_window_t<float, DCV, DRV>(p, s);
  MLA_ROPE_CASE(192, 32)
  MLA_ROPE_CASE(128, 32)
  MLA_ROPE_CASE(160, 64)
  MLA_ROPE_CASE(192, 64)
  MLA_ROPE_CASE(16, 8)
#undef MLA_ROPE_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_flash(int dtype, int d_c, int d_rope, const FlashParams& p, bool split, bool causal,
                        hipStream_t s) {
  if (p.Mb <= 0 || p.batch <= 0 || p.grid <= 0) return hipSuccess;
#define MLA_FLASH_CASE(DCV, DRV)                                                                  \
  if (d_c == DCV && d_rope == DRV)                                                                \
    return dtype == 0 ? launch_flash_t<bf16, DCV, DRV>(p, split, causal, s)                       \
                      : launch_flash_t<float, DCV, DRV>(p, split, causal, s);
  MLA_FLASH_CASE(192, 32)
  MLA_FLASH_CASE(128, 32)
  MLA_FLASH_CASE(160, 64)
  MLA_FLASH_CASE(192, 64)
  MLA_FLASH_CASE(16, 8)
#undef MLA_FLASH_CASE
  return hipErrorInvalidValue;
}

}  // namespace mla
