// Cache write (hyper.ai summary of VideoMLA, Method section): each token is
// projected once to its content latent c = W_dkv x and its unrotated
// positional key kR = W_kR x, and the row [c | kR] is stored into the
// sliding-window ring (chatpaper.ai abstract: fixed-size window), frame f in
// slot f mod W.
//
// GEMM view: out[r][n] = sum_k x[r][k] * Wcat[n][k], Wcat = [W_dkv ; W_kR]
// (N = d_c + d_rope). The step is bound by HBM: every x byte is read once
// from memory and 14x fewer bytes are written.
//
// bf16 with hidden = 1536 (the Wan2.1-1.3B width): work-group tiles of 80
// token rows x 64 outputs (236 tiles for a 3-frame Wan chunk, all resident
// at once). Both operands stream through LDS in 128-wide K steps with direct
// global->LDS loads, two steps in flight through four stage buffers; each
// staged row is 256 bytes and its 16-byte chunks are XOR-permuted by the row
// index so the 16 rows that a matrix-core operand read touches hit different
// banks. The four waves split the tile 2 x 2 (two or three 16-row blocks by
// two 16-column blocks). A wave reads the operands of the next K step into
// a second register set while the products of the current one run, one
// read between two products, so that the LDS and the matrix cores of a
// compute unit work at the same time (the barrier of each step keeps the
// waves in step, so with reads and products in separate phases the whole
// unit alternated between the two). The output tile goes through LDS once
// more so that rows leave in 16-byte stores.
//
// Other shapes (fp32, small latents, other widths) use a plain kernel
// with 64 x 32 tiles and operands loaded straight from global memory.
#include "mla_common.hpp"
#include "mla_internal.hpp"

namespace mla {

namespace {
constexpr int kRowsPerBlock = 64;
constexpr int kColsPerBlock = 32;

// staged bf16 kernel
constexpr int kSM = 80;                           // token rows per tile (5 x 16)
constexpr int kSN = 64;                           // outputs per tile (4 x 16, one block per wave)
constexpr int kSK = 128;                          // K per stage
constexpr int kSChunks = kSK * 2 / 16;            // 16-byte chunks per staged row (16)
constexpr int kSRows = kSM + kSN;                 // staged rows per stage
constexpr int kSInstr = kSRows * kSChunks / 64;   // direct-load instructions per stage (36)
constexpr int kSInstrWave = (kSInstr + 3) / 4;    // per wave (9)
constexpr int kSElems = kSRows * kSK;             // bf16 elements per stage buffer
constexpr int kSOutLd = kSN + 8;                  // output staging row stride (elements)
static_assert(kSRows * kSChunks % 64 == 0, "whole direct-load instructions per stage");
static_assert(kSM * kSOutLd <= kSElems, "output staging fits in one stage buffer");
static_assert(2 * kSInstrWave < 64, "vmcnt range");
static_assert(4 * kSElems * 2 <= 160 * 1024, "four stage buffers fit in LDS");
}  // namespace

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// The same, and also until this wave's LDS operations have all returned.
template <int N>
__device__ __forceinline__ void wait_vm_lds() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
}

// XCD-major order: consecutive logical tiles (which share token rows) land on
// one XCD, whose L2 then serves the repeated x reads.
__device__ __forceinline__ int xcd_logical(int id, int per_xcd) { return (id % kXcds) * per_xcd + id / kXcds; }

// One wave's share of the K loop: NMB row blocks from rb0 on by the two
// column blocks from column 32 wc on. Four stage buffers; iteration s waits
// for this wave's loads of stage s + 1 (stage s + 2 may stay in flight),
// meets the other waves at a barrier (every wave's loads of s + 1 have
// landed, and every wave has finished the products of s - 1, whose buffer
// stage s + 3 now takes), starts stage s + 3, and then reads the operands of
// s + 1 into one register set while the products of s run from the other,
// reads and products interleaved one for one so that the LDS and the matrix
// cores work at the same time. The barrier is the bare instruction: a full
// __syncthreads() would also wait for every outstanding load. The stage
// loop is unrolled completely (NSTAGE is a template parameter) so that every
// buffer is known at compile time and the compiler adds no waits of its own
// for the loads still in flight.
template <int NSTAGE, int NMB, typename Issue>
__device__ __forceinline__ void staged_loop(bool active, int wc, int rb0, Issue& issue, bf16* sb0, bf16* sb1,
                                            bf16* sb2, bf16* sb3, f32x4 (&acc)[3][2]) {
  const int lane = threadIdx.x & 63, li = lane & 15, lg = lane >> 4;
  struct Ops {
    bf16x8 b[kSK / 32][2], a[kSK / 32][NMB];
  };
  // staged row r, logical chunk c -> element (r * kSChunks + (c ^ (r % kSChunks))) * 8
  auto read_ops = [&](const bf16* buf, Ops& o) {
#pragma unroll
    for (int kc = 0; kc < kSK / 32; ++kc) {
      const int c = kc * 4 + lg;
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const int rb = kSM + wc * 32 + cb * 16 + li;
        o.b[kc][cb] = load8<bf16>(buf + (rb * kSChunks + (c ^ (rb & (kSChunks - 1)))) * 8);
      }
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) {
        const int ra = (rb0 + mb) * 16 + li;
        o.a[kc][mb] = load8<bf16>(buf + (ra * kSChunks + (c ^ (ra & (kSChunks - 1)))) * 8);
      }
    }
  };
  auto products = [&](const Ops& o) {
#pragma unroll
    for (int kc = 0; kc < kSK / 32; ++kc)
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) acc[mb][cb] = mma16(o.a[kc][mb], o.b[kc][cb], acc[mb][cb]);
  };
  constexpr int kReads = (kSK / 32) * (2 + NMB), kProducts = (kSK / 32) * NMB * 2;
  auto buf = [&](int i) -> bf16* { return i == 0 ? sb0 : i == 1 ? sb1 : i == 2 ? sb2 : sb3; };
  Ops ops[2];
#pragma unroll
  for (int s = 0; s < 3 && s < NSTAGE; ++s) issue(s, buf(s));
  if (NSTAGE >= 3)
    wait_vm<2 * kSInstrWave>();
  else if (NSTAGE == 2)
    wait_vm<kSInstrWave>();
  else
    wait_vm<0>();
  __builtin_amdgcn_s_barrier();
  if (active) read_ops(buf(0), ops[0]);
#pragma unroll
  for (int s = 0; s < NSTAGE; ++s) {
    if (s + 1 < NSTAGE) {
      // the LDS reads of stage s, issued one iteration ago, are waited for
      // here too, where they have long returned: a count of 15 cannot say
      // "all but the reads issued next", so a wait the compiler placed among
      // the products would wait for those as well
      if (s + 2 < NSTAGE)
        wait_vm_lds<kSInstrWave>();
      else
        wait_vm_lds<0>();
      __builtin_amdgcn_s_barrier();
      if (s + 3 < NSTAGE) issue(s + 3, buf((s + 3) % 4));
      if (active) {
        read_ops(buf((s + 1) % 4), ops[(s + 1) & 1]);
        products(ops[s & 1]);
        // one read, one product, ... then the reads left over
#pragma unroll
        for (int i = 0; i < kProducts; ++i) {
          if (i < kReads) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
        if (kReads > kProducts) __builtin_amdgcn_sched_group_barrier(0x100, kReads - kProducts, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    } else if (active) {
      products(ops[s & 1]);
    }
  }
}

template <int NSTAGE>
__global__ __launch_bounds__(256) void cache_write_staged_kernel(CacheWriteParams p, int n_tiles_n, int n_logical,
                                                                 int per_xcd) {
  __shared__ __attribute__((aligned(16))) bf16 sb0[kSElems];
  __shared__ __attribute__((aligned(16))) bf16 sb1[kSElems];
  __shared__ __attribute__((aligned(16))) bf16 sb2[kSElems];
  __shared__ __attribute__((aligned(16))) bf16 sb3[kSElems];
  const int logical = xcd_logical(blockIdx.x, per_xcd);
  if (logical >= n_logical) return;
  const int row0 = (logical / n_tiles_n) * kSM;
  const int col0 = (logical % n_tiles_n) * kSN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int n_out = p.d_c + p.d_rope;

  if (logical == 0) {
    for (int e = tid; e < p.batch * p.n_frames; e += blockDim.x) {
      const int b = e / p.n_frames, f = p.frame_first + e % p.n_frames;
      p.slot_frame[b * p.W + f % p.W] = f;
    }
  }

  // direct-load sources: instruction k of this wave fills LDS chunks
  // [64 i, 64 i + 64), i = wave + 4k; chunk q of staged row sr holds global
  // chunk q ^ (sr % kSChunks) of that row. Rows past the end repeat the last row.
  const char* src[kSInstrWave];
  int dst_off[kSInstrWave];
#pragma unroll
  for (int k = 0; k < kSInstrWave; ++k) {
    const int instr = min(wave + 4 * k, kSInstr - 1);
    const int pos = instr * 64 + lane;
    const int sr = pos / kSChunks, c = (pos % kSChunks) ^ (sr & (kSChunks - 1));
    const bf16* rowp;
    if (sr < kSM) {
      rowp = (const bf16*)p.x + (size_t)min(row0 + sr, p.rows - 1) * p.hidden;
    } else {
      const int n = min(col0 + sr - kSM, n_out - 1);
      rowp = n < p.d_c ? (const bf16*)p.w_dkv + (size_t)n * p.hidden
                       : (const bf16*)p.w_kr + (size_t)(n - p.d_c) * p.hidden;
    }
    src[k] = (const char*)(rowp + c * 8);
    dst_off[k] = instr * 64 * 8;  // elements
  }
  // Work-groups walk K from different starting steps, so the many tiles that
  // share W rows (and the few that share x rows) do not all ask the L2 for
  // the same lines at the same moment. The sum is the same in any order.
  const int k_start = logical % NSTAGE;
  auto issue = [&](int stage, bf16* buf) {
    int ks = stage + k_start;
    ks = ks >= NSTAGE ? ks - NSTAGE : ks;
#pragma unroll
    for (int k = 0; k < kSInstrWave; ++k)
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src[k] + ks * kSK * 2),
                                       (MLA_LDS void*)(MLA_LDS bf16*)(buf + dst_off[k]), 16, 0, 0);
  };

  // Waves in 2 x 2: wave w takes outputs 32 (w & 1) .. + 32 (two 16-column
  // blocks) of row blocks 0-1 (w < 2) or 2-4 (w >= 2).
  const int wr = wave >> 1, wc = wave & 1;
  const int rb0 = wr == 0 ? 0 : 2;
  const bool active = col0 + wc * 32 < n_out;  // this wave's outputs exist
  f32x4 acc[3][2] = {};
  if (wr == 0)
    staged_loop<NSTAGE, 2>(active, wc, rb0, issue, sb0, sb1, sb2, sb3, acc);
  else
    staged_loop<NSTAGE, 3>(active, wc, rb0, issue, sb0, sb1, sb2, sb3, acc);

  // output tile -> LDS (bf16) -> 16-byte stores of whole row segments
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  bf16* ot = sb0;
  if (active) {
    const int nmb = wr == 0 ? 2 : 3;
#pragma unroll
    for (int mb = 0; mb < 3; ++mb)
      if (mb < nmb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            ot[((rb0 + mb) * 16 + lg * 4 + i) * kSOutLd + wc * 32 + cb * 16 + li] = (bf16)acc[mb][cb][i];
  }
  __syncthreads();
  const int n_cols = min(kSN, n_out - col0);  // a multiple of 8
  for (int e = tid; e < kSM * (kSN / 8); e += 256) {
    const int r = e / (kSN / 8), c8 = (e % (kSN / 8)) * 8;
    const int row = row0 + r;
    if (row >= p.rows || c8 >= n_cols) continue;
    const int b = row / p.rows_per_b, local = row - b * p.rows_per_b;
    const int f = p.frame_first + local / p.T, tok = local % p.T;
    bf16* dst = (bf16*)p.cache + (((size_t)b * p.W + f % p.W) * p.T + tok) * n_out + col0 + c8;
    *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(ot + r * kSOutLd + c8);
  }
}

// Writes of many tokens (a window prefill, a chunk of many streams): tiles
// of 128 token rows x all outputs, so that every x row is read from memory
// by one work-group only, and W (at most 0.8 MB, the same for every tile)
// is served by the L2. Four waves in 2 x 2: 64 rows x NCB 16-output blocks
// each. 64-wide K steps through three LDS stage buffers (two in flight),
// direct global->LDS loads, 16-byte chunks XOR-permuted by row; the
// output tile leaves through LDS in 16-byte row pieces.
namespace {
constexpr int kWM = 128;                            // token rows per tile
constexpr int kWK = 64;                             // K per stage
constexpr int kWChunks = kWK * 2 / 16;              // 16-byte chunks per staged row (8)
}  // namespace

template <int NSTAGE, int NCB>
__global__ __launch_bounds__(256) void cache_write_wide_kernel(CacheWriteParams p, int n_logical, int per_xcd) {
  constexpr int WN = 2 * NCB * 16;                  // outputs (= d_c + d_rope)
  constexpr int ROWS = kWM + WN;                    // staged rows per stage
  constexpr int INSTR = ROWS * kWChunks / 64;       // direct-load instructions per stage
  constexpr int INSTR_WAVE = (INSTR + 3) / 4;
  constexpr int ELEMS = INSTR * 64 * 8;             // bf16 per stage buffer (whole instructions)
  constexpr int OLD = WN + 8;                       // output staging row stride
  static_assert(ROWS * kWChunks % 64 == 0, "whole direct-load instructions per stage");
  static_assert((kWM / 2) * OLD <= ELEMS, "half the output tile fits in one stage buffer");
  static_assert(INSTR_WAVE < 32, "two stages of loads within the vmcnt range");
  __shared__ __attribute__((aligned(16))) bf16 wb0[ELEMS];
  __shared__ __attribute__((aligned(16))) bf16 wb1[ELEMS];
  __shared__ __attribute__((aligned(16))) bf16 wb2[ELEMS];
  const int logical = xcd_logical(blockIdx.x, per_xcd);
  if (logical >= n_logical) return;
  const int row0 = logical * kWM;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int wr = wave >> 1, wc = wave & 1;

  if (logical == 0) {
    for (int e = tid; e < p.batch * p.n_frames; e += blockDim.x) {
      const int b = e / p.n_frames, f = p.frame_first + e % p.n_frames;
      p.slot_frame[b * p.W + f % p.W] = f;
    }
  }

  // instruction i fills staged rows 8 i .. 8 i + 7; lane L writes row
  // 8 i + L / 8, LDS chunk L % 8, which holds global chunk (L % 8) ^ (L / 8)
  const char* src[INSTR_WAVE];
  int dst_off[INSTR_WAVE];
#pragma unroll
  for (int k = 0; k < INSTR_WAVE; ++k) {
    const int instr = min(wave + 4 * k, INSTR - 1);
    const int sr = instr * 8 + (lane >> 3), c = (lane & 7) ^ (lane >> 3);
    const bf16* rowp;
    if (sr < kWM) {
      rowp = (const bf16*)p.x + (size_t)min(row0 + sr, p.rows - 1) * p.hidden;
    } else {
      const int n = sr - kWM;
      rowp = n < p.d_c ? (const bf16*)p.w_dkv + (size_t)n * p.hidden
                       : (const bf16*)p.w_kr + (size_t)(n - p.d_c) * p.hidden;
    }
    src[k] = (const char*)(rowp + c * 8);
    dst_off[k] = instr * 64 * 8;
  }
  const int k_start = logical % NSTAGE;  // staggered K order (W lines not all requested at once)
  auto issue = [&](int stage, bf16* buf) {
    int ks = stage + k_start;
    ks = ks >= NSTAGE ? ks - NSTAGE : ks;
#pragma unroll
    for (int k = 0; k < INSTR_WAVE; ++k)
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src[k] + ks * kWK * 2),
                                       (MLA_LDS void*)(MLA_LDS bf16*)(buf + dst_off[k]), 16, 0, 0);
  };

  f32x4 acc[4][NCB] = {};
  // staged row r, logical chunk c: element (r * 8 + (c ^ (r % 8))) * 8
  // all of a stage's operand reads first, then its products (one wave per
  // SIMD: nothing else hides the LDS latency)
  auto compute = [&](const bf16* buf) {
    bf16x8 aop[kWK / 32][4], bop[kWK / 32][NCB];
#pragma unroll
    for (int kc = 0; kc < kWK / 32; ++kc) {
      const int c = kc * 4 + lg;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const int ra = wr * 64 + mb * 16 + li;
        aop[kc][mb] = load8<bf16>(buf + (ra * kWChunks + (c ^ (ra & 7))) * 8);
      }
#pragma unroll
      for (int nb = 0; nb < NCB; ++nb) {
        const int rb = kWM + (wc * NCB + nb) * 16 + li;
        bop[kc][nb] = load8<bf16>(buf + (rb * kWChunks + (c ^ (rb & 7))) * 8);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kc = 0; kc < kWK / 32; ++kc)
#pragma unroll
      for (int nb = 0; nb < NCB; ++nb)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) acc[mb][nb] = mma16(aop[kc][mb], bop[kc][nb], acc[mb][nb]);
  };

  auto buf = [&](int i) -> bf16* { return i == 0 ? wb0 : i == 1 ? wb1 : wb2; };
  issue(0, buf(0));
  if (NSTAGE > 1) issue(1, buf(1));
#pragma unroll
  for (int s = 0; s < NSTAGE; ++s) {
    if (s + 1 < NSTAGE)
      wait_vm<INSTR_WAVE>();  // this stage's loads have landed, the next one's may not
    else
      wait_vm<0>();
    __builtin_amdgcn_s_barrier();
    if (s + 2 < NSTAGE) issue(s + 2, buf((s + 2) % 3));
    compute(buf(s % 3));
  }

  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // output rows 0..63 (wave row 0) staged in the first buffer, 64..127 in the second
  bf16* ot = wr == 0 ? wb0 : wb1;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < NCB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        ot[(mb * 16 + lg * 4 + i) * OLD + (wc * NCB + nb) * 16 + li] = (bf16)acc[mb][nb][i];
  __syncthreads();
  for (int e = tid; e < kWM * (WN / 8); e += 256) {
    const int r = e / (WN / 8), c8 = (e % (WN / 8)) * 8;
    const int row = row0 + r;
    if (row >= p.rows) continue;
    const int b = row / p.rows_per_b, local = row - b * p.rows_per_b;
    const int f = p.frame_first + local / p.T, tok = local % p.T;
    bf16* dst = (bf16*)p.cache + (((size_t)b * p.W + f % p.W) * p.T + tok) * WN + c8;
    const bf16* srcp = (r < kWM / 2 ? wb0 + r * OLD : wb1 + (r - kWM / 2) * OLD) + c8;
    *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(srcp);
  }
}

template <typename T>
__global__ __launch_bounds__(256) void cache_write_kernel(CacheWriteParams p, int n_tiles_n, int n_logical,
                                                          int per_xcd) {
  typedef typename V8<T>::type v8;
  const int id = blockIdx.x;
  const int logical = xcd_logical(id, per_xcd);
  if (logical >= n_logical) return;
  const int row_tile = logical / n_tiles_n;
  const int col_tile = logical % n_tiles_n;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int n_out = p.d_c + p.d_rope;

  if (logical == 0) {
    for (int e = tid; e < p.batch * p.n_frames; e += blockDim.x) {
      const int b = e / p.n_frames, f = p.frame_first + e % p.n_frames;
      p.slot_frame[b * p.W + f % p.W] = f;
    }
  }

  const int row = row_tile * kRowsPerBlock + wave * 16 + li;  // A-operand row of this lane
  const bool row_ok = row < p.rows;
  const T* xrow = (const T*)p.x + (size_t)(row_ok ? row : 0) * p.hidden;
  const T* wrow[2];
  bool col_ok[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int n = col_tile * kColsPerBlock + nb * 16 + li;
    col_ok[nb] = n < n_out;
    const int nn = col_ok[nb] ? n : 0;
    wrow[nb] = nn < p.d_c ? (const T*)p.w_dkv + (size_t)nn * p.hidden
                          : (const T*)p.w_kr + (size_t)(nn - p.d_c) * p.hidden;
  }

  f32x4 acc[2] = {};
  for (int k0 = 0; k0 < p.hidden; k0 += 32) {
    const int k = k0 + lg * 8;
    const bool k_ok = k < p.hidden;
    const v8 a = (row_ok && k_ok) ? load8<T>(xrow + k) : zero8<T>();
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const v8 b = (col_ok[nb] && k_ok) ? load8<T>(wrow[nb] + k) : zero8<T>();
      acc[nb] = mma16(a, b, acc[nb]);
    }
  }

  // lane holds out[4*lg + i][16*nb + li] of this wave's 16 x 32 block
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = row_tile * kRowsPerBlock + wave * 16 + lg * 4 + i;
    if (r >= p.rows) continue;
    const int b = r / p.rows_per_b, local = r % p.rows_per_b;
    const int f = p.frame_first + local / p.T, tok = local % p.T;
    T* dst = (T*)p.cache + (((size_t)b * p.W + f % p.W) * p.T + tok) * n_out;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int n = col_tile * kColsPerBlock + nb * 16 + li;
      if (n < n_out) dst[n] = to_t<T>(acc[nb][i]);
    }
  }
}

hipError_t launch_cache_write(int dtype, int d_c, int d_rope, const CacheWriteParams& p, hipStream_t s) {
  (void)d_c;
  (void)d_rope;
  const int n_out = p.d_c + p.d_rope;
  // many tokens: tiles over all outputs from 96 tiles of 128 rows on (x is
  // read once; a work-group's K loop takes about the same time at any size,
  // so below that the narrower tiles, spread over every compute unit, finish
  // first; measured crossover between 74 and 110 tiles)
  if (dtype == 0 && p.hidden == 1536 && (p.rows + kWM - 1) / kWM >= 96 &&
      (n_out == 224 || n_out == 160 || n_out == 256)) {
    const int n_logical = (p.rows + kWM - 1) / kWM;
    const int per_xcd = (n_logical + kXcds - 1) / kXcds;
    const dim3 grid(per_xcd * kXcds);
    if (n_out == 224)
      hipLaunchKernelGGL((cache_write_wide_kernel<1536 / kWK, 7>), grid, dim3(256), 0, s, p, n_logical, per_xcd);
    else if (n_out == 160)
      hipLaunchKernelGGL((cache_write_wide_kernel<1536 / kWK, 5>), grid, dim3(256), 0, s, p, n_logical, per_xcd);
    else
      hipLaunchKernelGGL((cache_write_wide_kernel<1536 / kWK, 8>), grid, dim3(256), 0, s, p, n_logical, per_xcd);
    return hipGetLastError();
  }
  if (dtype == 0 && p.hidden == 1536 && n_out % 8 == 0 && p.rows >= 1) {
    const int n_tiles_n = (n_out + kSN - 1) / kSN;
    const int n_logical = ((p.rows + kSM - 1) / kSM) * n_tiles_n;
    const int per_xcd = (n_logical + kXcds - 1) / kXcds;
    hipLaunchKernelGGL(cache_write_staged_kernel<1536 / kSK>, dim3(per_xcd * kXcds), dim3(256), 0, s, p, n_tiles_n,
                       n_logical, per_xcd);
    return hipGetLastError();
  }
  const int n_tiles_n = (n_out + kColsPerBlock - 1) / kColsPerBlock;
  const int n_tiles_m = (p.rows + kRowsPerBlock - 1) / kRowsPerBlock;
  const int n_logical = n_tiles_m * n_tiles_n;
  const int per_xcd = (n_logical + kXcds - 1) / kXcds;
  const int grid = per_xcd * kXcds;
  if (dtype == 0)
    hipLaunchKernelGGL(cache_write_kernel<bf16>, dim3(grid), dim3(256), 0, s, p, n_tiles_n, n_logical, per_xcd);
  else
    hipLaunchKernelGGL(cache_write_kernel<float>, dim3(grid), dim3(256), 0, s, p, n_tiles_n, n_logical, per_xcd);
  return hipGetLastError();
}

}  // namespace mla
