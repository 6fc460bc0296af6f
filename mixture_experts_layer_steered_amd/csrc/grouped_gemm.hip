// Grouped expert GEMMs of the routed-MoE layer on gfx950 (CDNA4) bf16 MFMA.
//
// One launch per projection covers every expert (and the shared expert in
// the same launch) -- "Module glm5next_mlp", Modules forward_prefill_gemm:
// one grouped launch per projection for all experts, with tile variants.
//
//   gate_up: per group g and row r of its segment,
//            [g_r, u_r] = A[row(r)] @ W_gu[g]^T (fp32 accumulators), and the
//            epilogue writes h[r] = bf16(silu(min(g_r, L)) * clamp(u_r, -L, L))
//            -- the clamp of "Numerics the kernels rely on", applied to the
//            fp32 accumulators.  A workgroup owns BN gate columns and the
//            matching BN up columns (rows n and I + n of the fused weight,
//            "mstar.model.components.distributed.mlp", ParallelGatedMLP), so
//            each lane holds g and u of the same (row, column) in the same
//            accumulator slot.
//   down:    y[r] = h[r] @ W_d[g]^T, fp32 out.
//
// Operands are K-contiguous on both sides ([rows, K] activations, [out, in]
// weights), so every lane feeds the MFMA with one 16-byte LDS read per
// operand fragment.  Tiles are staged through LDS (BK = 64, 16-byte chunks
// XOR-swizzled by row to spread banks) with a register prefetch of the next
// K step in flight during the MFMAs.  Rows of a routed tile are gathered
// through row_index (the permutation), so no permuted copy of x is made.
//
// Schedule: expert segment sizes live on the device.  A one-workgroup
// kernel turns group_offsets into the prefix of m-tiles per group; each GEMM
// workgroup maps its tile id to (group, m-tile, n-tile) by binary search and
// exits when past the end.  Workgroup ids are remapped so each of the 8 XCDs
// works a contiguous range of tiles, m-tiles fastest: consecutive tiles on an
// XCD share one weight n-tile in that XCD's L2.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace {

constexpr int BK = 64;
constexpr int CH = BK / 8;  // 16-byte chunks per LDS row

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ (row & 7); }

__device__ __forceinline__ int xcd_remap(int bid, int nb) {
  const int xcd = bid & 7, local = bid >> 3;
  const int per = nb >> 3, rem = nb & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + local;
}

// Uniform loads through the scalar data cache (waited on with lgkmcnt, so
// they never wait behind the direct-to-LDS stage loads and stores the way
// a vector load's vmcnt wait does).
__device__ __forceinline__ int32_t ws_sload(const int32_t* p, int64_t i) {
  return ((const __attribute__((address_space(4))) int32_t*)p)[i];
}
__device__ __forceinline__ float ws_sloadf(const float* p, int64_t i) {
  return ((const __attribute__((address_space(4))) float*)p)[i];
}

template <int BM, int BN, int WAVES_M, int WAVES_N, bool GATEUP>
__device__ __forceinline__ void gemm_tile(const GemmProblem& P, int tile, float limit) {
  constexpr int THREADS = WAVES_M * WAVES_N * 64;
  constexpr int NB = GATEUP ? 2 * BN : BN;  // weight rows per tile
  constexpr int WM = BM / WAVES_M;          // rows per wave
  constexpr int WN = BN / WAVES_N;          // output columns per wave
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int NMAT = GATEUP ? 2 : 1;
  constexpr int A_CHUNKS = BM * CH / THREADS;
  constexpr int B_CHUNKS = NB * CH / THREADS;
  static_assert(A_CHUNKS >= 1 && B_CHUNKS >= 1, "tile too small for the workgroup");
  static_assert(BM * CH % THREADS == 0 && NB * CH % THREADS == 0, "uneven load split");

  __shared__ __attribute__((aligned(16))) uint16_t As[BM * BK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[NB * BK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;

  const int mt_global = tile % P.max_mtiles;
  const int nt = tile / P.max_mtiles;

  // tile -> group, first row, end row
  int g = 0;
  int64_t row0, row_end;
  if (P.group_offsets == nullptr) {
    row0 = (int64_t)mt_global * BM;
    row_end = P.M;
    if (row0 >= row_end) return;
  } else {
    if (mt_global >= P.mtile_start[P.G]) return;
    int lo = 0, hi = P.G - 1;  // last g with mtile_start[g] <= mt_global
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if (P.mtile_start[mid] <= mt_global) lo = mid; else hi = mid - 1;
    }
    g = lo;
    row0 = P.group_offsets[g] + (int64_t)(mt_global - P.mtile_start[g]) * BM;
    row_end = P.group_offsets[g + 1];
  }
  const int n0 = nt * BN;
  const int K = P.K, N = P.N;
  const uint16_t* __restrict__ Wg = P.W + (int64_t)g * P.w_stride;

  // per-thread source rows of the A and B chunks it loads (fixed over K)
  const uint16_t* a_src[A_CHUNKS];
  int a_dst[A_CHUNKS];
  int a_cc[A_CHUNKS];
#pragma unroll
  for (int i = 0; i < A_CHUNKS; ++i) {
    const int c = tid + i * THREADS;
    const int r = c / CH, cc = c % CH;
    const int64_t gr = row0 + r;
    a_src[i] = nullptr;
    if (gr < row_end) {
      const int64_t src = P.row_index ? (int64_t)P.row_index[gr] : gr;
      a_src[i] = P.A + src * K + cc * 8;
    }
    a_dst[i] = r * BK + swz(r, cc) * 8;
    a_cc[i] = cc;
  }
  const uint16_t* b_src[B_CHUNKS];
  int b_dst[B_CHUNKS];
  int b_cc[B_CHUNKS];
#pragma unroll
  for (int i = 0; i < B_CHUNKS; ++i) {
    const int c = tid + i * THREADS;
    const int r = c / CH, cc = c % CH;
    int n, wrow;
    if (GATEUP) {
      n = n0 + (r < BN ? r : r - BN);
      wrow = r < BN ? n : N + n;  // gate rows [0, N), up rows [N, 2N)
    } else {
      n = n0 + r;
      wrow = n;
    }
    b_src[i] = (n < N) ? Wg + (int64_t)wrow * K + cc * 8 : nullptr;
    b_dst[i] = r * BK + swz(r, cc) * 8;
    b_cc[i] = cc;
  }

  f32x16_t acc[NMAT][TM][TN];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[m][i][j][r] = 0.f;

  uint4 a_reg[A_CHUNKS], b_reg[B_CHUNKS];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) {
      a_reg[i] = make_uint4(0, 0, 0, 0);
      if (a_src[i] && k0 + a_cc[i] * 8 < K) a_reg[i] = *reinterpret_cast<const uint4*>(a_src[i] + k0);
    }
#pragma unroll
    for (int i = 0; i < B_CHUNKS; ++i) {
      b_reg[i] = make_uint4(0, 0, 0, 0);
      if (b_src[i] && k0 + b_cc[i] * 8 < K) b_reg[i] = *reinterpret_cast<const uint4*>(b_src[i] + k0);
    }
  };

  load(0);
  for (int k0 = 0; k0 < K; k0 += BK) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) *reinterpret_cast<uint4*>(&As[a_dst[i]]) = a_reg[i];
#pragma unroll
    for (int i = 0; i < B_CHUNKS; ++i) *reinterpret_cast<uint4*>(&Bs[b_dst[i]]) = b_reg[i];
    __syncthreads();
    if (k0 + BK < K) load(k0 + BK);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int chunk = ks * 2 + (lane >> 5);
      bf16x8_t af[TM];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = wm * WM + i * 32 + (lane & 31);
        af[i] = *reinterpret_cast<const bf16x8_t*>(&As[r * BK + swz(r, chunk) * 8]);
      }
#pragma unroll
      for (int m = 0; m < NMAT; ++m) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int r = m * BN + wn * WN + j * 32 + (lane & 31);
          const bf16x8_t bfrag = *reinterpret_cast<const bf16x8_t*>(&Bs[r * BK + swz(r, chunk) * 8]);
#pragma unroll
          for (int i = 0; i < TM; ++i)
            acc[m][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfrag, acc[m][i][j], 0, 0, 0);
        }
      }
    }
  }

  // epilogue: 32x32 accumulator, lane holds column (lane & 31) and rows
  // 8*(r/4) + 4*(lane/32) + r%4; the group's output scale (1 without one)
  // multiplies the fp32 sums first
  const float ts = P.tscale ? ws_sloadf(P.tscale, g) : 1.0f;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = n0 + wn * WN + j * 32 + (lane & 31);
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = row0 + wm * WM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row >= row_end) continue;
        if (GATEUP) {
          const float hv =
              swiglu_clamped(acc[0][i][j][r] * ts, acc[NMAT - 1][i][j][r] * ts, limit);
          static_cast<uint16_t*>(P.out)[row * N + col] = (uint16_t)f32_to_bf16_bits(hv);
        } else {
          static_cast<float*>(P.out)[row * N + col] = acc[0][i][j][r] * ts;
        }
      }
    }
  }
}

template <int BM, int BN, int WAVES_M, int WAVES_N, bool GATEUP>
__global__ __launch_bounds__(WAVES_M * WAVES_N * 64) void grouped_gemm_kernel(
    GemmProblem p0, GemmProblem p1, int tiles0, float limit) {
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  if (tile < tiles0)
    gemm_tile<BM, BN, WAVES_M, WAVES_N, GATEUP>(p0, tile, limit);
  else
    gemm_tile<BM, BN, WAVES_M, WAVES_N, GATEUP>(p1, tile - tiles0, limit);
}

constexpr int PL_MBLK = 8;

// ---------------------------------------------------------------------------
// Pipelined LDS-tiled variant for long expert segments (prefill).
//
// Persistent: one workgroup per CU walks a dense list of output tiles.  The
// real tile count is read on the device (m-tile prefix x n-tiles, routed
// and shared problems back to back) and split into 8 equal contiguous
// ranges, one per XCD (workgroup b runs on XCD b % 8), so every XCD gets the
// same work and its 32 CUs work on neighbouring tiles that share A and B
// rows in its L2.  Inside a problem tiles run group (expert) major, then in
// blocks of up to 8 m-tiles, n-tile, m-tile: the m-tiles of an expert (a few
// in prefill) that use one weight tile run side by side and read it from HBM
// once, and an expert's weights go to one XCD.
//
// Workgroup tile: BM rows x BN output columns (gate_up: BN gate + BN up
// weight rows), eight wavefronts as 2 x 4, each owning (BM/2) x (BN/4)
// outputs (x2 for gate/up) in 32x32 MFMA accumulators (weight fragment as
// the first operand, so a lane holds runs of four adjacent output columns
// for one A row and the epilogue stores 8 or 16 bytes at a time).  K
// advances KB at a time through STAGES LDS slots filled by direct
// buffer->LDS 16-byte loads (buffer_load_dwordx4 ... lds), STAGES-1 of them
// in flight.  A row of a stage is KB*2 bytes; each load instruction writes
// 1 KB of LDS in lane order (1024/(KB*2) whole rows), and the XOR swizzle
// of the 16-byte chunk slots -- chosen so the 16 rows one ds_read_b128 pass
// touches fall in 16 different bank groups of the 64-bank LDS -- comes from
// which global chunk each lane fetches.  Rows past a segment or past N
// fetch the tile's first row (their products reach only outputs never
// stored).
//
// Two schedules of the same tile: interleaved (below, the else branch of
// pipe_tile) and ping-pong (the PP branch).  Interleaved, per step: the
// MFMAs of K substep s run while the fragments of substep s+1 are read from
// LDS; the loads of the stage STAGES-1 ahead go out with the first substep;
// before the last substep each wave waits for its own loads of the next
// stage and its own LDS reads, then a fence-free barrier makes the next
// stage visible (its substep-0 fragments are read during the last
// substep's MFMAs).

__device__ __forceinline__ void lds_direct_16(const void* g, uint16_t* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_wave_base, 16,
                                   0, 0);
}

// The same for data read exactly once (streamed expert weights): the
// non-temporal policy keeps the stream from displacing reused lines and lets
// HBM deliver more of its rate (decode gate_up: 222 -> 211 us for 1.41 GB).
__device__ __forceinline__ void lds_direct_16_stream(const void* g, uint16_t* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_wave_base, 16,
                                   0, 2 /* nt */);
}

// Raw buffer resource over [base, base + 4 GiB): stride 0, the largest record
// count, and the dword-3 word of CDNA's untyped buffer loads.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t pl_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, -1, 0x00020000);
}

// 16 bytes per lane from rsrc at voff + soff bytes into LDS, lane L's bytes at
// lds_wave_base + 16 L (buffer_load_dwordx4 ... lds)
__device__ __forceinline__ void lds_buffer_16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff,
                                              uint32_t soff, uint16_t* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rsrc, (__attribute__((address_space(3))) void*)lds_wave_base, 16, voff, soff, 0, 0);
}

// s_waitcnt vmcnt(n) with lgkmcnt(0) (gfx9 encoding: vmcnt[3:0] and [15:14],
// expcnt[6:4], lgkmcnt[11:8]): this wave's loads up to the n newest and all of
// its LDS reads and writes have completed.
#define PL_WAIT_VM_LDS(n) __builtin_amdgcn_s_waitcnt((((n) & 15) | (((n) >> 4) << 14)) | 0x0070)
#define PL_WAIT_VM(n) __builtin_amdgcn_s_waitcnt((((n) & 15) | (((n) >> 4) << 14)) | 0x0F70)
// lgkmcnt(0) alone: this wave's LDS reads and writes have completed
#define PL_WAIT_LDS() __builtin_amdgcn_s_waitcnt(0xC07F)
// vmcnt(n) with lgkmcnt(m), m < 16: all but this wave's m newest LDS
// operations have completed (they complete in order)
#define PL_WAIT_VM_LDS_N(n, m) \
  __builtin_amdgcn_s_waitcnt((((n) & 15) | (((n) >> 4) << 14)) | 0x0070 | ((m) << 8))

// Workgroup barrier without a memory fence.  __syncthreads() fences, which
// makes every wave wait for all of its outstanding loads (including the
// direct-to-LDS loads of later stages) and would drain the pipeline at each
// step.  Here the waits are explicit (PL_WAIT_VM_LDS before the barrier) and
// the empty asm statements only stop the compiler from moving memory
// operations across the barrier.
__device__ __forceinline__ void pl_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int KB>
__device__ __forceinline__ int pl_swz(int row, int chunk) {
  // 64-byte rows: 4 rows share a 256-byte bank cycle; 128-byte rows: 2 rows
  return KB == 32 ? chunk ^ ((row >> 2) & 3) : chunk ^ ((row >> 1) & 7);
}

// Compile-time shape of the pipelined tile; PACKED: the weights in the
// tile-blocked layout of launch_pack_experts; HBLK: h stage-blocked within
// each tile (gate_up writes it so, down reads it so as its A): the tile's
// rows [row0, row0 + rows) of K columns keep their row-major footprint,
// holding stage s (columns [32 s, 32 s + 32)) of row r at element
// row0 * K + (s * rows + r) * 32.
template <int BM_, int BN_, bool GATEUP_, int KB_, int NW_, int WAVES_M_, bool PACKED_ = false,
          bool HBLK_ = false>
struct PipeShape {
  static constexpr int BM = BM_, BN = BN_, KB = KB_, NW = NW_, WAVES_M = WAVES_M_;
  static constexpr bool GATEUP = GATEUP_, PACKED = PACKED_, HBLK = HBLK_;
  static constexpr int NB = GATEUP ? 2 * BN : BN;  // weight rows per tile
  static constexpr int ROWS = BM + NB;             // LDS rows per stage
  static constexpr int CHUNKS = KB / 8;            // 16-byte chunks per row
  static constexpr int STAGE = ROWS * KB;          // bf16 elements per stage
  static constexpr int RPI = 64 / CHUNKS;          // rows per 1 KB load instruction
  static constexpr int INSTR = ROWS / RPI;         // load instructions per stage
  static constexpr int PER_WAVE = INSTR / NW;      // of them per wavefront
  static constexpr int WAVES_N = NW / WAVES_M;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int TM = WM / 32, TN = WN / 32;
  static constexpr int NMAT = GATEUP ? 2 : 1;
  static constexpr int SUB = KB / 16;              // MFMA K substeps per stage
  static constexpr int A_INSTR = BM / (NW * RPI);  // instructions of each wave that fill A rows
  static constexpr int STORES = TM * TN * 4;       // epilogue stores per wave
  static_assert(INSTR % NW == 0 && SUB % 2 == 0, "shape");
  static_assert(BM % (NW * RPI) == 0, "A rows fill whole instructions of every wave");
  static_assert(!PACKED || (KB == 32 && NB == 256), "the tile-blocked layout: 256 x 32 blocks");
  static_assert(!HBLK || KB == 32, "h blocks of 32 columns");
  // bytes between the K stages of one weight row: 64 in rows of K, one
  // 256 x 32 block tile-blocked
  static constexpr uint32_t W_STAGE = PACKED ? NB * KB * 2 : KB * 2;
};

// One output tile as one wavefront sees it: rows [row0, row_end) of its
// problem (one group's segment), output columns from n0, and the per-lane
// byte offsets of this wave's load instructions from two buffer resources
// (A, and this group's weights).
template <class S>
struct PipeTile {
  int64_t row0, row_end;
  int n0;
  float ts;  // the group's output scale (1 without one)
  __amdgpu_buffer_rsrc_t rs_a, rs_w;
  uint32_t off[S::PER_WAVE];
};

// Rows of tile T (BM, fewer in a segment's last tile).
template <class S>
__device__ __forceinline__ int64_t pipe_rows(const PipeTile<S>& T) {
  return T.row_end - T.row0 < S::BM ? T.row_end - T.row0 : S::BM;
}

// Tile t of a problem with mt_total m-tiles.  Tile order: group (expert)
// major, then blocks of up to PL_MBLK m-tiles, n-tile, m-tile (the last
// block of a group may be narrower).  Instruction i of wave w fills stage
// rows RPI*q .. RPI*q+RPI-1 with q = w + NW*i; lane L writes row
// RPI*q + L/CHUNKS, slot L%CHUNKS, which holds logical chunk pl_swz(row,
// slot) (the swizzle is an involution).  Rows past the segment or past N
// fetch the tile's first row (their products reach only outputs never
// stored).  Offsets are 32-bit: A and one group's weights hold fewer than
// 2^31 elements (the host checks).
//
// pipe_coords: the tile's rows, first column, output scale and A resource;
// returns its group.
template <class S>
__device__ __forceinline__ int pipe_coords(const GemmProblem& P, int mt_total, int tile,
                                           PipeTile<S>& T) {
  int g = 0, ms = 0, mc = mt_total;
  if (P.group_offsets != nullptr) {
    int lo = 0, hi = P.G - 1;  // last g with mtile_start[g] * ntiles <= tile
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if (ws_sload(P.mtile_start, mid) * P.ntiles <= tile) lo = mid; else hi = mid - 1;
    }
    g = lo;
    ms = ws_sload(P.mtile_start, g);
    mc = ws_sload(P.mtile_start, g + 1) - ms;
  }
  const int local = tile - ms * P.ntiles;
  const int blk = local / (PL_MBLK * P.ntiles);
  const int rem = local - blk * PL_MBLK * P.ntiles;
  const int width = min(PL_MBLK, mc - blk * PL_MBLK);
  const int nt = rem / width;
  const int ml = blk * PL_MBLK + rem % width;
  T.row0 = (P.group_offsets ? (int64_t)ws_sload(P.group_offsets, g) : 0) + (int64_t)ml * S::BM;
  T.row_end = P.group_offsets ? (int64_t)ws_sload(P.group_offsets, g + 1) : P.M;
  T.n0 = nt * S::BN;
  T.ts = P.tscale ? ws_sloadf(P.tscale, g) : 1.0f;
  T.rs_a = pl_rsrc(P.A);
  return g;
}

// Row of the A piece that lane `lane` of load instruction i of wave `wave`
// fetches, in the problem's row space (clamped to the tile's first row past
// the segment).
template <class S>
__device__ __forceinline__ int32_t pipe_a_row(const PipeTile<S>& T, int i, int wave, int lane) {
  const int row = S::RPI * (wave + S::NW * i) + lane / S::CHUNKS;
  return (int32_t)(T.row0 + row < T.row_end ? T.row0 + row : T.row0);
}

// Byte offset of that piece, from its source row in A.
template <class S>
__device__ __forceinline__ uint32_t pipe_a_off_of(int K, int32_t a_row, int i, int wave,
                                                  int lane) {
  const int row = S::RPI * (wave + S::NW * i) + lane / S::CHUNKS;
  const int chunk = pl_swz<S::KB>(row, lane % S::CHUNKS);
  return (uint32_t)(((int64_t)a_row * K + chunk * 8) * 2);
}

// Tile T's place in three parts.  pipe_locate_coords: coordinates, weight
// offsets, and the A rows in the problem's row space (in T.off[i <
// A_INSTR]); pipe_locate_rows: those rows through row_index when A is
// gathered (per-lane vector loads, which may still be in flight after it;
// measured: reading the rows through the scalar cache instead, 16 loads and
// selects per instruction, was slower); pipe_locate_end: the rows to byte
// offsets.  Between the last two the caller can run steps whose waits see
// the row loads land, so that no wait for them drains the stage loads and
// stores issued before them.
template <class S>
__device__ __forceinline__ void pipe_locate_coords(const GemmProblem& P, int mt_total, int tile,
                                                   PipeTile<S>& T) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = pipe_coords<S>(P, mt_total, tile, T);
  T.rs_w = pl_rsrc(P.W + (int64_t)g * P.w_stride);
  const int K = P.K, N = P.N;
#pragma unroll
  for (int i = 0; i < S::PER_WAVE; ++i) {
    const int row = S::RPI * (wave + S::NW * i) + lane / S::CHUNKS;
    const int chunk = pl_swz<S::KB>(row, lane % S::CHUNKS);
    if (i < S::A_INSTR) {
      T.off[i] = (uint32_t)pipe_a_row<S>(T, i, wave, lane);
    } else if constexpr (S::PACKED) {
      // tile-blocked weights: tile row r's 32 values of stage s at byte
      // ((tile * K/32 + s) * NB + r) * 64; the stage part goes in the
      // scalar offset (pipe_issue)
      const int r = row - S::BM;
      T.off[i] = (uint32_t)((int64_t)(T.n0 / S::BN) * S::NB * K * 2 + r * 64 + chunk * 16);
    } else {
      const int r = row - S::BM;
      int n = S::GATEUP ? T.n0 + (r < S::BN ? r : r - S::BN) : T.n0 + r;
      const bool up = S::GATEUP && r >= S::BN;
      if (n >= N) n = T.n0;
      T.off[i] = (uint32_t)(((int64_t)(up ? N + n : n) * K + chunk * 8) * 2);
    }
  }
}

template <class S>
__device__ __forceinline__ void pipe_locate_rows(const int32_t* row_index, PipeTile<S>& T) {
  if (row_index != nullptr) {
#pragma unroll
    for (int i = 0; i < S::A_INSTR; ++i) T.off[i] = (uint32_t)row_index[T.off[i]];
  }
}

template <class S>
__device__ __forceinline__ void pipe_locate_end(int K, PipeTile<S>& T) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int i = 0; i < S::A_INSTR; ++i) {
    if constexpr (S::HBLK && !S::GATEUP) {
      // A stage-blocked within the tile: the row's 64 bytes of stage 0 at
      // row0 * K * 2 + r * 64; the stage part goes in the scalar offset
      const int row = S::RPI * (wave + S::NW * i) + lane / S::CHUNKS;
      const int chunk = pl_swz<S::KB>(row, lane % S::CHUNKS);
      T.off[i] = (uint32_t)(T.row0 * K * 2 + ((int64_t)T.off[i] - T.row0) * 64 + chunk * 16);
    } else {
      T.off[i] = pipe_a_off_of<S>(K, (int32_t)T.off[i], i, wave, lane);
    }
  }
}

template <class S>
__device__ __forceinline__ void pipe_locate(const GemmProblem& P, int mt_total, int tile,
                                            PipeTile<S>& T) {
  pipe_locate_coords<S>(P, mt_total, tile, T);
  pipe_locate_rows<S>(P.row_index, T);
  pipe_locate_end<S>(P.K, T);
}

// This wave's loads of the K columns [k0, k0 + KB) of tile T into LDS slot
// `slot` (K is a multiple of KB here, so every stage is whole).
template <class S>
__device__ __forceinline__ void pipe_issue(const PipeTile<S>& T, uint16_t* smem, int slot,
                                           int k0) {
  const int wave = threadIdx.x >> 6;
  uint16_t* base = smem + slot * S::STAGE;
  // bytes between A's K stages: 64 in rows of K; the tile's rows x 64 when
  // stage-blocked
  uint32_t a_soff = (uint32_t)k0 * 2;
  if constexpr (S::HBLK && !S::GATEUP) a_soff = (uint32_t)(k0 / S::KB) * (uint32_t)pipe_rows(T) * 64u;
#pragma unroll
  for (int i = 0; i < S::PER_WAVE; ++i)
    lds_buffer_16(i < S::A_INSTR ? T.rs_a : T.rs_w, T.off[i],
                  i < S::A_INSTR ? a_soff : (uint32_t)(k0 / S::KB) * S::W_STAGE,
                  base + (wave + S::NW * i) * S::RPI * S::KB);
}

// Quad permutation of a float across each group of four lanes (DPP).
template <int CTRL>
__device__ __forceinline__ float quad_dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// 4x4 transpose inside each quad of lanes: afterwards register r of lane b
// (b = lane % 4) holds what register b of lane r held.  Two butterfly steps,
// each exchanging one bit of the lane index with the same bit of the register
// index: a lane sends its partner (lane ^ 1, then lane ^ 2) the one register
// of each pair the partner needs, picked by its own lane bit, so each step
// takes two DPP moves.  Written out without a loop: the loop form of the same
// steps was compiled into a single move per step, with wrong results.
__device__ __forceinline__ void quad_transpose(f32x4_t& v) {
  const int lane = threadIdx.x & 63;
  const bool b0 = lane & 1, b1 = lane & 2;
  const float x0 = quad_dpp<0xB1>(b0 ? v[0] : v[1]);  // lanes 1,0,3,2
  const float x1 = quad_dpp<0xB1>(b0 ? v[2] : v[3]);
  const float t0 = b0 ? x0 : v[0], t1 = b0 ? v[1] : x0;
  const float t2 = b0 ? x1 : v[2], t3 = b0 ? v[3] : x1;
  const float y0 = quad_dpp<0x4E>(b1 ? t0 : t2);      // lanes 2,3,0,1
  const float y1 = quad_dpp<0x4E>(b1 ? t1 : t3);
  v[0] = b1 ? y0 : t0;
  v[1] = b1 ? y1 : t1;
  v[2] = b1 ? t2 : y0;
  v[3] = b1 ? t3 : y1;
}

// One 32x32x16 MFMA of the tile.  In gate_up the weight fragment is the
// first operand, so an accumulator is a 32 (weight rows) x 32 (A rows) block
// and a lane holds one A row: it owns both g and u of four runs of four
// adjacent output columns, which the clamped SwiGLU pairs up in registers.
// In down the A fragment goes first: a lane then holds one output column of
// 16 A rows, so a quad of lanes holds 4x4 blocks of y that a transpose turns
// into rows; a 16-byte store of the wave then writes 8 whole 128-byte row
// pieces instead of 32-byte pieces of 32 rows (the fp32 epilogue of this
// tile writes 256 KB).
template <class S>
__device__ __forceinline__ f32x16_t pipe_mfma(const bf16x8_t& w, const bf16x8_t& a,
                                              const f32x16_t& c) {
  if constexpr (S::GATEUP)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(w, a, c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, w, c, 0, 0, 0);
}

// Epilogue.  gate_up: lane L holds A row L % 32 and weight rows
// 8*(r/4) + 4*(L/32) + r%4 of its 32x32 block, i.e. four runs of four
// adjacent output columns -- 8-byte stores of h.  N is a multiple of 32
// here, so a run is either wholly inside N or past it.  down: lane L holds
// output column L % 32 of A rows 8*(r/4) + 4*(L/32) + r%4 -- one dword of y
// per register, turned into four adjacent columns of one row by a quad
// transpose (lane 4a+b: row 8*g + 4*(L/32) + b, columns 4a..4a+3 of the
// block, for each group g of four registers).
//
// The stores are buffer stores through a resource that spans exactly the
// tile's rows of the output ([row0, min(row_end, row0 + BM)) x N): lanes
// past the segment fall outside it, lanes past N are sent outside it, and
// the buffer range check drops both.  So every wave issues exactly
// S::STORES stores for every tile, and the stage waits right after an
// epilogue can count them (pipe offsets stay below 2^31: N <= 2^20, which
// the host checks).  (wm, wn): the wave's row half and column block.
// (The resource's fields go through readfirstlane: they are uniform, and a
// resource the compiler cannot prove uniform costs a loop around every
// store.)
template <class S>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t pipe_out_rsrc(const GemmProblem& P,
                                                                const PipeTile<S>& T) {
  constexpr int ES = S::GATEUP ? 2 : 4;  // bytes per output element
  const int64_t rows = pipe_rows(T);
  const uint64_t base = reinterpret_cast<uint64_t>(static_cast<char*>(P.out) + T.row0 * P.N * ES);
  const uint64_t b = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(base >> 32)) << 32) |
                     (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)base);
  const int nrec = __builtin_amdgcn_readfirstlane((int)(rows * P.N * ES));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(b), (short)0, nrec, 0x00020000);
}

// One epilogue store at byte offset `off` of resource rs.  The offset passes
// through an empty asm statement so that the compiler can neither merge nor
// drop stores (several go to the same dropped offset): the stage waits after
// an epilogue count exactly S::STORES of them.
__device__ __forceinline__ void pipe_st64(uint2_t v, __amdgpu_buffer_rsrc_t rs, uint32_t off) {
  asm volatile("" : "+v"(off));
  __builtin_amdgcn_raw_buffer_store_b64(v, rs, off, 0, 0);
}
__device__ __forceinline__ void pipe_st128(f32x4_t v, __amdgpu_buffer_rsrc_t rs, uint32_t off) {
  asm volatile("" : "+v"(off));
  __builtin_amdgcn_raw_buffer_store_b128(v, rs, off, 0, 0);
}

template <class S, bool HALF = false>
__device__ __forceinline__ void pipe_store(const GemmProblem& P, const PipeTile<S>& T,
                                           const f32x16_t (&acc)[S::NMAT][S::TM][S::TN],
                                           float limit, int wm, int wn) {
  const int lane = threadIdx.x & 63;
  const int N = P.N;
  const __amdgpu_buffer_rsrc_t rs = pipe_out_rsrc<S>(P, T);
  constexpr uint32_t kOut = 0x80000000u;  // past every tile's resource
  // a half-height tile (HALF): the wave's rows start at wm WM/2 and only
  // its first TM/2 row blocks hold sums; the others' stores are dropped
  constexpr int WROWS = HALF ? S::WM / 2 : S::WM;
  auto live = [](int i) { return !HALF || i < S::TM / 2; };
  if constexpr (S::GATEUP) {
    const uint32_t rows = (uint32_t)pipe_rows(T);
#pragma unroll
    for (int i = 0; i < S::TM; ++i) {
      const int r = wm * WROWS + i * 32 + (lane & 31);
#pragma unroll
      for (int j = 0; j < S::TN; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = T.n0 + wn * S::WN + j * 32 + 8 * q + 4 * (lane >> 5);
          const f32x16_t& g = acc[0][i][j];
          const f32x16_t& u = acc[S::NMAT - 1][i][j];
          const float ts = T.ts;
          float2_t h01 = {swiglu_clamped_fast(g[4 * q] * ts, u[4 * q] * ts, limit),
                          swiglu_clamped_fast(g[4 * q + 1] * ts, u[4 * q + 1] * ts, limit)};
          float2_t h23 = {swiglu_clamped_fast(g[4 * q + 2] * ts, u[4 * q + 2] * ts, limit),
                          swiglu_clamped_fast(g[4 * q + 3] * ts, u[4 * q + 3] * ts, limit)};
          uint2_t pk = {__builtin_bit_cast(uint32_t, __builtin_convertvector(h01, bf16x2_t)),
                        __builtin_bit_cast(uint32_t, __builtin_convertvector(h23, bf16x2_t))};
          // stage-blocked h: row r of stage col / 32 at (col / 32 * rows + r) * 64
          // bytes (rows past the segment would land in other rows: dropped)
          const uint32_t off = S::HBLK ? ((uint32_t)(col >> 5) * rows + r) * 64u + (col & 31) * 2u
                                       : (uint32_t)(r * N + col) * 2u;
          pipe_st64(pk, rs,
                    live(i) && col < N && (!S::HBLK || (uint32_t)r < rows) ? off : kOut);
        }
      }
    }
  } else {
    // registers 4g..4g+3 hold a 4 (rows) x 1 (column) piece; the four lanes
    // of a quad together hold a 4x4 block, which quad_transpose turns into
    // one row of four adjacent columns per lane
    const int quad = (lane & 31) >> 2;
#pragma unroll
    for (int i = 0; i < S::TM; ++i)
#pragma unroll
      for (int j = 0; j < S::TN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4_t v = {acc[0][i][j][4 * g] * T.ts, acc[0][i][j][4 * g + 1] * T.ts,
                       acc[0][i][j][4 * g + 2] * T.ts, acc[0][i][j][4 * g + 3] * T.ts};
          quad_transpose(v);
          const int r = wm * WROWS + i * 32 + 8 * g + 4 * (lane >> 5) + (lane & 3);
          const int col = T.n0 + wn * S::WN + j * 32 + 4 * quad;
          pipe_st128(v, rs, live(i) && col < N ? (uint32_t)(r * N + col) * 4u : kOut);
        }
  }
}

// The same number of stores as pipe_store, all dropped (an empty resource):
// stands in for the epilogue of the tile before a workgroup's first, so that
// the first tile's stage waits count the same queue as every later tile's.
template <class S>
__device__ __forceinline__ void pipe_store_none(const GemmProblem& P) {
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(P.out, (short)0, 0, 0x00020000);
#pragma unroll
  for (int q = 0; q < S::STORES; ++q) {
    if constexpr (S::GATEUP)
      pipe_st64(uint2_t{0u, 0u}, rs, 0u);
    else
      pipe_st128(f32x4_t{0.f, 0.f, 0.f, 0.f}, rs, 0u);
  }
}

template <class S>
__device__ __forceinline__ void pipe_zero(f32x16_t (&acc)[S::NMAT][S::TM][S::TN]) {
#pragma unroll
  for (int m = 0; m < S::NMAT; ++m)
#pragma unroll
    for (int i = 0; i < S::TM; ++i)
#pragma unroll
      for (int j = 0; j < S::TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[m][i][j][r] = 0.f;
}

// One tile, interleaved schedule (both wavefronts of a SIMD read fragments
// and issue MFMAs; one barrier per stage).
template <class S, int STAGES>
__device__ __forceinline__ void pipe_tile(const GemmProblem& P, int mt_total, int tile,
                                          float limit, uint16_t* smem) {
  constexpr int BM = S::BM, BN = S::BN, KB = S::KB;
  constexpr int STAGE = S::STAGE, TM = S::TM, TN = S::TN, NMAT = S::NMAT, SUB = S::SUB;
  constexpr int WM = S::WM, WN = S::WN;
  constexpr int VM_STAGE = S::PER_WAVE;  // vector memory instructions per stage per wave
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave / S::WAVES_N, wn = wave % S::WAVES_N;

  PipeTile<S> T;
  pipe_locate<S>(P, mt_total, tile, T);
  const int nk = P.K / KB;
  auto stage_k = [&](int s) __attribute__((always_inline)) { return min(s, nk - 1) * KB; };
  auto issue = [&](int slot, int k0) __attribute__((always_inline)) {
    pipe_issue<S>(T, smem, slot, k0);
  };

  f32x16_t acc[NMAT][TM][TN];
  pipe_zero<S>(acc);

  // MFMA fragments of one 16-wide K substep, two groups (substeps alternate)
  bf16x8_t af[2][TM], bfr[2][NMAT][TN];
  auto read_frags = [&](int slot, int ks, auto grp_c) __attribute__((always_inline)) {
    constexpr int grp = decltype(grp_c)::value;
    const uint16_t* As = smem + slot * STAGE;
    const uint16_t* Bs = As + BM * KB;
    const int chunk = ks * 2 + (lane >> 5);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int r = wm * WM + i * 32 + (lane & 31);
      af[grp][i] = *reinterpret_cast<const bf16x8_t*>(&As[r * KB + pl_swz<KB>(r, chunk) * 8]);
    }
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int r = m * BN + wn * WN + j * 32 + (lane & 31);
        bfr[grp][m][j] = *reinterpret_cast<const bf16x8_t*>(&Bs[r * KB + pl_swz<KB>(r, chunk) * 8]);
      }
  };
  auto mfmas = [&](auto grp_c) __attribute__((always_inline)) {
    constexpr int grp = decltype(grp_c)::value;
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int i = 0; i < TM; ++i)
          acc[m][i][j] = pipe_mfma<S>(bfr[grp][m][j], af[grp][i], acc[m][i][j]);
  };
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  constexpr int NREAD = TM + NMAT * TN;  // fragment reads per substep
  constexpr int NMFMA = TM * NMAT * TN;  // MFMAs per substep
  // Every step issues exactly one stage of loads (stages past the end
  // re-fetch the last K step into a free slot).  With four or more slots the
  // loads of step kt refill the slot of stage kt-2 (LAG 2), else that of
  // stage kt-1 (LAG 1); AHEAD = STAGES - LAG stages are issued ahead of the
  // one being read, so "stage kt+1 landed" is "at most AHEAD-1 newer stages
  // of this wave's loads in flight".  Before the barrier of step kt each wave
  // also finishes its reads of the slot the next step refills: with LAG 2
  // those are all but its newest NREAD reads (the fragments of the substep
  // still to come), so the wait does not stall on reads just issued; with
  // LAG 1 all of them.
  constexpr int LAG = STAGES >= 4 ? 2 : 1;
  constexpr int AHEAD = STAGES - LAG;

  // every wave done reading LDS (the previous tile's last stage) before the
  // slots are refilled.  No fence: the previous tile's loads all landed
  // before its epilogue, and its epilogue stores drain while this tile's
  // first stages load (they are only older entries of the vmcnt queue in the
  // waits below)
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  pl_barrier();
#pragma unroll
  for (int s0 = 0; s0 < AHEAD; ++s0) issue(s0, stage_k(s0));
  PL_WAIT_VM_LDS((AHEAD - 1) * VM_STAGE);
  pl_barrier();
  read_frags(0, 0, C0{});

  int slot = 0;            // LDS slot of stage kt
  int slot_issue = AHEAD;  // slot of stage kt + AHEAD
  for (int kt = 0; kt < nk; ++kt) {
    const int slot_next = slot + 1 == STAGES ? 0 : slot + 1;
#pragma unroll
    for (int ks = 0; ks < SUB; ++ks) {
      const bool even = (ks & 1) == 0;
      if (ks == SUB - 1) {
        // own loads of stage kt+1 landed, own reads of the slot the next
        // step refills done: after the barrier stage kt+1 is complete
        // everywhere and nobody still reads that slot
        if (LAG == 2)
          PL_WAIT_VM_LDS_N((AHEAD - 1) * VM_STAGE, NREAD);
        else
          PL_WAIT_VM_LDS((AHEAD - 1) * VM_STAGE);
        pl_barrier();
      }
      // read the fragments of the next substep, then the MFMAs of substep
      // ks.  In this program order both fragment groups are live at once, so
      // they keep separate registers (reads placed after the MFMAs let the
      // register allocator fold the groups into one).
      if (ks + 1 < SUB) {
        if (even) read_frags(slot, ks + 1, C1{}); else read_frags(slot, ks + 1, C0{});
      } else {
        read_frags(slot_next, 0, C0{});
      }
      if (even) mfmas(C0{}); else mfmas(C1{});
      if (ks == 0) issue(slot_issue, stage_k(kt + AHEAD));
      // schedule: the first MFMA (its operands were read a substep ago, so
      // its wait finds them done), then all fragment reads of the next
      // substep, then the remaining MFMAs with the stage loads spread
      // between them
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, NREAD, 0);
#pragma unroll
      for (int q = 1; q < NMFMA; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (ks == 0 && q <= VM_STAGE) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
      if (ks == 0 && NMFMA <= VM_STAGE)
        __builtin_amdgcn_sched_group_barrier(0x020, VM_STAGE - NMFMA + 1, 0);
    }
    slot = slot_next;
    slot_issue = slot_issue + 1 == STAGES ? 0 : slot_issue + 1;
  }
  // the re-fetches past the end of K landed: nothing of this tile is still
  // in flight into LDS when the next tile refills the slots
  PL_WAIT_VM(0);
  pipe_store<S>(P, T, acc, limit, wm, wn);
}

template <int BM>
__device__ __forceinline__ int pipe_mtiles(const GemmProblem& P) {
  return P.group_offsets ? P.mtile_start[P.G] : (int)((P.M + BM - 1) / BM);
}

// Persistent: one workgroup per CU.  The real tile counts are read on the
// device (m-tile prefix x n-tiles; routed problem, then shared problem) and
// each problem is split into 8 equal contiguous ranges, one per XCD
// (workgroup b runs on XCD b % 8): an XCD takes its share of the routed
// tiles, then its share of the shared expert's.  Its workgroups stride that
// sequence (virtual index v, tile(v) the real tile).  Splitting the
// concatenated tile list instead gave one XCD all of the shared expert's
// tiles, which differ in cost (ScMoE: twice the K in down, no partly filled
// m-tiles), and that XCD ended last by up to half the launch.
struct PipeRange {
  int mt0, mt1, tiles0, t_first, t_end, stride;
  int base0, n0, base1;  // this XCD's first routed tile and count, first shared tile
  __device__ __forceinline__ int tile(int v) const { return v < n0 ? base0 + v : base1 + (v - n0); }
};
template <int BM>
__device__ __forceinline__ PipeRange pipe_range(const GemmProblem& p0, const GemmProblem& p1,
                                                int has_p1) {
  PipeRange R;
  R.mt0 = pipe_mtiles<BM>(p0);
  R.mt1 = has_p1 ? pipe_mtiles<BM>(p1) : 0;
  R.tiles0 = R.mt0 * p0.ntiles;
  const int tiles1 = R.mt1 * p1.ntiles;
  const int nwg = gridDim.x, b = blockIdx.x;
  const int xcd = b & 7, lid = b >> 3;
  R.stride = (nwg - xcd + 7) >> 3;
  R.base0 = (int)((int64_t)R.tiles0 * xcd / 8);
  R.n0 = (int)((int64_t)R.tiles0 * (xcd + 1) / 8) - R.base0;
  R.base1 = R.tiles0 + (int)((int64_t)tiles1 * xcd / 8);
  const int n1 = R.tiles0 + (int)((int64_t)tiles1 * (xcd + 1) / 8) - R.base1;
  R.t_first = lid;
  R.t_end = R.n0 + n1;
  return R;
}

template <class S, int STAGES>
__global__ __launch_bounds__(S::NW * 64, 1) void grouped_pipe_kernel(GemmProblem p0,
                                                                     GemmProblem p1, int has_p1,
                                                                     float limit) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem_dyn[];
  const PipeRange R = pipe_range<S::BM>(p0, p1, has_p1);
  for (int v = R.t_first; v < R.t_end; v += R.stride) {
    const int t = R.tile(v);
    if (t < R.tiles0)
      pipe_tile<S, STAGES>(p0, R.mt0, t, limit, smem_dyn);
    else
      pipe_tile<S, STAGES>(p1, R.mt1, t - R.tiles0, limit, smem_dyn);
  }
}

// Ping-pong schedule of the same tile (eight wavefronts as two groups of
// four, wave w on SIMD w % 4, so each SIMD holds one wave of each group).
// Group 0 owns the tile's first BM/2 rows, group 1 the rest.  A step of one
// group is a memory phase -- read the fragments of one K stage from LDS,
// issue this wave's share of the stage AHEAD = STAGES-1 ahead, wait for its
// own loads of the next stage -- then a barrier, then the compute phase (the
// stage's MFMAs from registers only), then a barrier.  Group 1 runs one
// barrier behind group 0 for the whole launch, so on every SIMD one wave
// computes while the other reads and loads.
//
// The stage stream runs on across the workgroup's tiles: the last AHEAD
// steps of a tile issue the first stages of its next tile (whose place is
// computed at the tile's start), so a new tile starts on landed data and
// the epilogue of one group overlaps the other group's compute phase.  Stage
// s of the stream uses slot s % STAGES; stage s+STAGES refills the slot of
// stage s, and its loads go out in the memory phases of step s+1, after the
// barrier that ends group 1's memory phase of step s.  Every step issues one
// stage (past the last tile, the last stage again), so "the next stage
// landed" is always "at most AHEAD-1 newer stages of this wave's loads in
// flight" (the first AHEAD-1 steps of a tile also allow for the previous
// tile's epilogue stores, see `step`).  Needs K >= 2 AHEAD KB for every
// problem (the host checks).
template <class S, int STAGES>
__global__ __launch_bounds__(S::NW * 64, 1) void grouped_pp_kernel(GemmProblem p0, GemmProblem p1,
                                                                   int has_p1, float limit) {
  static_assert(S::NW == 8 && S::WAVES_M == 2, "two row halves, one per group");
  static_assert(S::KB == 32, "one 32-wide K stage per step");
  constexpr int KB = S::KB, BM = S::BM, BN = S::BN, STAGE = S::STAGE;
  constexpr int TM = S::TM, TN = S::TN, NMAT = S::NMAT, WM = S::WM, WN = S::WN;
  constexpr int AHEAD = STAGES - 1, VM_STAGE = S::PER_WAVE;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem_dyn[];
  uint16_t* smem = smem_dyn;
  const PipeRange R = pipe_range<BM>(p0, p1, has_p1);
  int v = R.t_first;  // position in this XCD's tile sequence
  if (v >= R.t_end) return;  // no tile for this workgroup (uniform)
  int t = R.tile(v);

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave / S::WAVES_N, wn = wave % S::WAVES_N;
  // the wave's group in a scalar register: barriers are only ever skipped
  // by whole wavefronts
  const int group = __builtin_amdgcn_readfirstlane(wave >> 2);

  // (the compiler merges the two branches' row loads into one; passing the
  // selected problem's row_index to a single call instead made it keep the
  // tiles in scratch memory)
  auto locate_begin = [&](int tt, PipeTile<S>& T) __attribute__((always_inline)) {
    if (tt < R.tiles0) {
      pipe_locate_coords<S>(p0, R.mt0, tt, T);
      pipe_locate_rows<S>(p0.row_index, T);
    } else {
      pipe_locate_coords<S>(p1, R.mt1, tt - R.tiles0, T);
      pipe_locate_rows<S>(p1.row_index, T);
    }
  };
  auto locate_end = [&](int tt, PipeTile<S>& T) __attribute__((always_inline)) {
    pipe_locate_end<S>(tt < R.tiles0 ? p0.K : p1.K, T);
  };
  auto stages_of = [&](int tt) __attribute__((always_inline)) {
    return (tt < R.tiles0 ? p0.K : p1.K) / KB;
  };

  f32x16_t acc[NMAT][TM][TN];
  bf16x8_t fa[2][TM], fb[2][NMAT][TN];
  // A tile of at most BM/2 rows (an expert's last m-tile, often) runs as a
  // half-height tile: group g takes rows [g BM/4, (g+1) BM/4), each wave
  // its first TM/2 row blocks, so both groups' compute phases halve instead
  // of one group's going idle.  Its stage loads, waits and stores are those
  // of a full tile; every output sums its products in the same order.
  auto read_stage = [&](int slot, auto half_c) __attribute__((always_inline)) {
    constexpr bool HALF = decltype(half_c)::value;
    constexpr int TMH = HALF ? TM / 2 : TM, WMH = HALF ? WM / 2 : WM;
    const uint16_t* As = smem + slot * STAGE;
    const uint16_t* Bs = As + BM * KB;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int chunk = s * 2 + (lane >> 5);
#pragma unroll
      for (int i = 0; i < TMH; ++i) {
        const int r = wm * WMH + i * 32 + (lane & 31);
        fa[s][i] = *reinterpret_cast<const bf16x8_t*>(&As[r * KB + pl_swz<KB>(r, chunk) * 8]);
      }
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int r = m * BN + wn * WN + j * 32 + (lane & 31);
          fb[s][m][j] = *reinterpret_cast<const bf16x8_t*>(&Bs[r * KB + pl_swz<KB>(r, chunk) * 8]);
        }
    }
  };
  auto compute = [&](auto half_c) __attribute__((always_inline)) {
    constexpr int TMH = decltype(half_c)::value ? TM / 2 : TM;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int i = 0; i < TMH; ++i)
            acc[m][i][j] =
                pipe_mfma<S>(fb[s][m][j], fa[s][i], acc[m][i][j]);
  };
  auto pp_barrier = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    pl_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  PipeTile<S> cur, nxt;
  locate_begin(t, cur);
  locate_end(t, cur);
  int nk = stages_of(t);
#pragma unroll
  for (int s0 = 0; s0 < AHEAD; ++s0) pipe_issue<S>(cur, smem, s0, s0 * KB);
  PL_WAIT_VM_LDS((AHEAD - 1) * VM_STAGE);
  pp_barrier();  // stage 0 complete everywhere
  if (group) pp_barrier();
  pipe_store_none<S>(p0);
  int slot = 0, slot_issue = AHEAD;
  // One step: read stage kt's fragments, issue this wave's loads of the
  // stage AHEAD ahead into the slot read in the step before (from tile src
  // at K offset k0), wait for its loads of stage kt+1, barrier, MFMAs,
  // barrier.  The waits of the first AHEAD-1 steps of a tile (RELAXED) let
  // the previous epilogue's S::STORES stores stay in flight: they were
  // issued after stages 0..AHEAD-1 of this tile and before stage AHEAD, so
  // "stage kt+1 landed" is "at most (AHEAD-1) VM_STAGE + STORES newer
  // operations in flight" (the A row loads of the next tile, issued after
  // the stores, only make that stricter); from step AHEAD-1 on, the stage
  // waited for is younger than the stores.
  auto step = [&](const PipeTile<S>& src, int k0, auto relaxed_c, auto half_c)
                  __attribute__((always_inline)) {
    read_stage(slot, half_c);
    pipe_issue<S>(src, smem, slot_issue, k0);
    if constexpr (decltype(relaxed_c)::value)
      PL_WAIT_VM_LDS((AHEAD - 1) * VM_STAGE + S::STORES);
    else
      PL_WAIT_VM_LDS((AHEAD - 1) * VM_STAGE);
    pp_barrier();
    compute(half_c);
    pp_barrier();
    slot = slot + 1 == STAGES ? 0 : slot + 1;
    slot_issue = slot_issue + 1 == STAGES ? 0 : slot_issue + 1;
  };
  using T0 = std::integral_constant<bool, false>;
  using T1 = std::integral_constant<bool, true>;
  for (;;) {
    const bool more = v + R.stride < R.t_end;
    const int t_next = more ? R.tile(v + R.stride) : t;
    // the next tile's A rows load while this tile's first AHEAD steps run
    // (their stages are this tile's: nk >= 2 AHEAD); the offsets are formed
    // after step AHEAD-1, whose wait has seen the rows land.  The last AHEAD
    // steps issue the next tile's first stages -- past the last tile, this
    // tile's first stages again, into slots nothing reads any more.
    if (more) locate_begin(t_next, nxt);
    pipe_zero<S>(acc);
    auto run = [&](auto half_c) __attribute__((always_inline)) {
#pragma unroll
      for (int kt = 0; kt < AHEAD - 1; ++kt) step(cur, (kt + AHEAD) * KB, T1{}, half_c);
      step(cur, (2 * AHEAD - 1) * KB, T0{}, half_c);
      if (more)
        locate_end(t_next, nxt);
      else
        nxt = cur;
      for (int kt = AHEAD; kt < nk - AHEAD; ++kt) step(cur, (kt + AHEAD) * KB, T0{}, half_c);
#pragma unroll 1
      for (int q = 0; q < AHEAD; ++q) step(nxt, q * KB, T0{}, half_c);
      pipe_store<S, decltype(half_c)::value>(t < R.tiles0 ? p0 : p1, cur, acc, limit, wm, wn);
    };
    if (cur.row_end - cur.row0 <= BM / 2)
      run(T1{});
    else
      run(T0{});
    if (!more) break;
    v += R.stride;
    t = t_next;
    nk = stages_of(t);
    cur = nxt;
  }
  // pairs with group 1's last barrier
  if (group == 0) pp_barrier();
}

// ---------------------------------------------------------------------------
// Ping-pong tile with W4A16 weights (long expert segments: the grouped
// W4A16 expert GEMM of "Module glm5next_mlp", in this library's format --
// see the weight-streaming W4A16 kernel below for the code and scale
// layout).
//
// The bf16 ping-pong above with the weights read as 4-bit codes and
// dequantised inside the tile.  A stages keep only the A rows (16 KB, five
// slots, four in flight); the weights arrive per 128-column group (four
// stages): each weight row's 64 code bytes and its E4M3 scale byte, two
// groups resident.  The two wave groups split the tile by columns here, not
// by rows: group g owns output columns [g BN/2, (g+1) BN/2) (wave w: column
// block 2 (w/4) + w%2 of four, row half (w/2)%2), so it needs only its own
// half of the weight rows -- and loads only that half, so that everything a
// group reads from a code slot was loaded, and waited for, by its own
// waves.  In its compute phase of stage s a group dequantises its half of
// stage s+1 into a two-slot bf16 ring -- one fma per weight,
// (128 + u) s - 136 s = (u - 8) s, exact in fp32 and, with at most 8
// significant bits, exact as the bf16 that its upper half is -- between its
// MFMAs; the barrier that ends the phase makes the ring slot visible to the
// group's memory phase of stage s+1, which reads the weight fragments from
// the ring.  The scale bytes are decoded through a 256-entry table of
// (s, -136 s) built in LDS at the start.
//
// Loads: every wave issues two A instructions per stage (the stage AHEAD
// ahead) and, at the first stage of each code group, first three more: its
// group's share of the next code group (two of 16 rows x 64 contiguous
// bytes each, the four 16-byte pieces of a row in XOR-swizzled positions so
// that a stage's reads of 16 consecutive rows hit 64 banks, and the group's
// 128 scale bytes).  That group's slot was last read in the compute phase
// two steps earlier, and its first stage is dequantised three steps later,
// after the wait that sees the A stage issued behind it land.  The wait for
// "the next A stage landed" leaves 9 loads in flight, or 6 when no code
// group was issued in the last three steps (stage index 3 mod 4), plus the
// previous epilogue's stores in a tile's first three steps.  The tensor
// scale multiplies the accumulators in the epilogue.  K must be a multiple
// of 128 and at least 256.
template <class S>
struct PpW4Layout {
  static constexpr int STAGES = 5;                         // A slots
  static constexpr int AHEAD = STAGES - 1;
  static constexpr int A_BYTES = S::BM * S::KB * 2;        // one A stage
  static constexpr int G_COLS = 128;                       // K columns of a code group
  static constexpr int G_STAGES = G_COLS / S::KB;          // stages per code group
  static constexpr int C_ROW = G_COLS / 2;                 // code bytes per row and group
  static constexpr int HALF = S::NB / 2;                   // weight rows per wave group
  static constexpr int C_BYTES = S::NB * C_ROW;
  static constexpr int C_SLOT = C_BYTES + S::NB;           // + a scale byte per weight row
  static constexpr int C_SLOTS = 2;
  static constexpr int RING = S::NB * S::KB * 2;           // one stage of bf16 weights
  static constexpr int C_OFF = STAGES * A_BYTES;           // code slots
  static constexpr int R_OFF = C_OFF + C_SLOTS * C_SLOT;   // bf16 ring
  static constexpr int T_OFF = R_OFF + 2 * RING;           // scale table
  static constexpr int BYTES = T_OFF + 256 * 8;
  static constexpr int A_VM = S::A_INSTR;                  // A loads per wave and stage
  static constexpr int C_VM = 3;                           // code-group loads per wave
  static_assert(S::KB == 32 && G_STAGES == 4 && C_ROW == 64, "four 16-byte pieces per row");
  static_assert(S::NB == 256 && S::NW == 8 && S::A_INSTR == 2 && HALF == 128,
                "two code instructions of 16 rows per wave");
  static_assert(C_SLOT % 16 == 0 && BYTES <= 160 * 1024, "LDS");
};

// Wave w's tile position in the column split: (row half, column block).
__device__ __forceinline__ int pp_w4_wm(int wave) { return (wave >> 1) & 1; }
__device__ __forceinline__ int pp_w4_wn(int wave) { return 2 * (wave >> 2) + (wave & 1); }

// Local row l of wave group g's half (gate_up: its BN/2 gate rows, then the
// matching up rows; down: 128 consecutive rows) as a global weight row of
// tile column n0 (columns past N read column n0).
template <class S>
__device__ __forceinline__ int64_t pp_w4_wrow(const GemmProblem& P, int n0, int g, int l) {
  constexpr int Q = S::GATEUP ? S::BN / 2 : PpW4Layout<S>::HALF;
  const bool up = S::GATEUP && l >= Q;
  int n = n0 + Q * g + (up ? l - Q : l);
  if (n >= P.N) n = n0;
  return up ? (int64_t)P.N + n : n;
}

// XOR swizzle of a code row's four 16-byte pieces
__device__ __forceinline__ int pp_w4_cswz(int r) { return (r >> 2) & 3; }

// A tile as one wave of the W4A16 tile sees it: the bf16 tile's fields (A
// offsets in t.off[0..1]), this expert's code and scale resources, and the
// byte offsets of the wave's two code pieces (local rows 16 (q + 4 i) +
// lane/4 of its group's half, q = w % 4; piece lane%4 swizzled) and scale
// piece (lane < 8: local rows 16 lane .. +15).
template <class S>
struct PpW4Tile {
  PipeTile<S> t;
  __amdgpu_buffer_rsrc_t rs_s;
  uint32_t off_c0, off_c1, off_s;
};

// Everything but the A offsets, as pipe_locate_coords + pipe_locate_rows (the
// A source rows in T.t.off[i < A_INSTR], loads possibly in flight); then
// pipe_locate_end turns them into offsets.
template <class S>
__device__ __forceinline__ void pp_w4_locate_begin(const GemmProblem& P, int mt_total, int tile,
                                                   int wave, PpW4Tile<S>& T) {
  using L = PpW4Layout<S>;
  const int lane = threadIdx.x & 63;
  const int g = pipe_coords<S>(P, mt_total, tile, T.t);
#pragma unroll
  for (int i = 0; i < S::A_INSTR; ++i) T.t.off[i] = (uint32_t)pipe_a_row<S>(T.t, i, wave, lane);
  pipe_locate_rows<S>(P.row_index, T.t);
  T.t.rs_w = pl_rsrc(reinterpret_cast<const uint8_t*>(P.W) + (int64_t)g * P.w_stride * 2);
  T.rs_s = pl_rsrc(P.S + (int64_t)g * P.s_stride);
  const int grp = wave >> 2, q = wave & 3;
  uint32_t off[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int l = 16 * (q + 4 * i) + lane / 4;
    const int piece = (lane % 4) ^ pp_w4_cswz(L::HALF * grp + l);
    off[i] = (uint32_t)(pp_w4_wrow<S>(P, T.t.n0, grp, l) * (P.K / 2) + piece * 16);
  }
  T.off_c0 = off[0];
  T.off_c1 = off[1];
  T.off_s = (uint32_t)pp_w4_wrow<S>(P, T.t.n0, grp, 16 * (lane & 7));
}

// This wave's share of code group `cg` (local to tile T) into code slot
// `cslot`; wr_total is the weight rows of one expert (gate_up 2N, down N):
// the scale rows of one group.  The slot holds the rows in local order, wave
// group g's half at rows 128 g ..; its scale bytes likewise.
template <class S>
__device__ __forceinline__ void pp_w4_issue_c(const PpW4Tile<S>& T, uint8_t* smem, int cslot,
                                              int cg, int wave, int wr_total) {
  using L = PpW4Layout<S>;
  const int lane = threadIdx.x & 63;
  const int grp = wave >> 2, q = wave & 3;
  uint8_t* base = smem + L::C_OFF + cslot * L::C_SLOT;
  lds_buffer_16(T.t.rs_w, T.off_c0, (uint32_t)cg * L::C_ROW,
                reinterpret_cast<uint16_t*>(base + (L::HALF * grp + 16 * q) * L::C_ROW));
  lds_buffer_16(T.t.rs_w, T.off_c1, (uint32_t)cg * L::C_ROW,
                reinterpret_cast<uint16_t*>(base + (L::HALF * grp + 16 * (q + 4)) * L::C_ROW));
  if (lane < 8)  // the group's four waves write the same 128 scale bytes
    lds_buffer_16(T.rs_s, T.off_s, (uint32_t)cg * (uint32_t)wr_total,
                  reinterpret_cast<uint16_t*>(base + L::C_BYTES + L::HALF * grp));
}

// This wave's A loads of stage k0 of tile T into A slot `slot`.
template <class S>
__device__ __forceinline__ void pp_w4_issue_a(const PpW4Tile<S>& T, uint8_t* smem, int slot,
                                              int k0, int wave) {
  using L = PpW4Layout<S>;
  uint8_t* base = smem + slot * L::A_BYTES;
#pragma unroll
  for (int i = 0; i < S::A_INSTR; ++i)
    lds_buffer_16(T.t.rs_a, T.t.off[i], (uint32_t)k0 * 2,
                  reinterpret_cast<uint16_t*>(base + (wave + S::NW * i) * S::RPI * S::KB * 2));
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Two weights (u - 8) s as one bf16 pair, from bytes j and j+1 of `nib`
// (a code in the low nibble of each; sel0 and sel1 pick them): each code
// becomes the fp32 128 + u (0x43 high byte, the code in the next byte), one
// fma with c = -136 s gives (u - 8) s exactly, and its upper half is the
// bf16 value; the pack takes the two upper halves.
__device__ __forceinline__ uint32_t w4_dequant2(uint32_t nib, uint32_t sel0, uint32_t sel1,
                                                float s, float c) {
  const float f0 = fmaf(__builtin_bit_cast(float, __builtin_amdgcn_perm(0x43434343u, nib, sel0)), s, c);
  const float f1 = fmaf(__builtin_bit_cast(float, __builtin_amdgcn_perm(0x43434343u, nib, sel1)), s, c);
  return __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, f1), __builtin_bit_cast(uint32_t, f0),
                               0x07060302u);
}
// byte j of a nibble word into byte 2 of an fp32 whose byte 3 is 0x43
constexpr uint32_t W4_SEL0 = 0x04000C0Cu, W4_SEL1 = 0x04010C0Cu, W4_SEL2 = 0x04020C0Cu,
                   W4_SEL3 = 0x04030C0Cu;

// MFMAs LO .. HI-1 of a stage, numbered in the order (substep, matrix,
// column block, row block): the two substeps' products into one accumulator
// are eight apart.  HALF: only those of the first TM/2 row blocks (a
// half-height tile).
template <class S, int LO, int HI, bool HALF = false>
__device__ __forceinline__ void pp_mfma_range(f32x16_t (&acc)[S::NMAT][S::TM][S::TN],
                                              const bf16x8_t (&fa)[2][S::TM],
                                              const bf16x8_t (&fb)[2][S::NMAT][S::TN]) {
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int m = 0; m < S::NMAT; ++m)
#pragma unroll
      for (int j = 0; j < S::TN; ++j)
#pragma unroll
        for (int i = 0; i < S::TM; ++i) {
          const int n = ((s * S::NMAT + m) * S::TN + j) * S::TM + i;
          if (n >= LO && n < HI && (!HALF || i < S::TM / 2))
            acc[m][i][j] = pipe_mfma<S>(fb[s][m][j], fa[s][i], acc[m][i][j]);
        }
}

template <class S>
__global__ __launch_bounds__(S::NW * 64, 1) void grouped_pp_w4_kernel(GemmProblem p0,
                                                                      float limit) {
  static_assert(S::NW == 8 && S::WAVES_M == 2 && S::KB == 32, "ping-pong shape");
  using L = PpW4Layout<S>;
  constexpr int KB = S::KB, BN = S::BN, STAGES = L::STAGES, AHEAD = L::AHEAD;
  constexpr int TM = S::TM, TN = S::TN, NMAT = S::NMAT, WM = S::WM, WN = S::WN;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem_dyn[];
  uint8_t* smem = reinterpret_cast<uint8_t*>(smem_dyn);
  uint16_t* ring = reinterpret_cast<uint16_t*>(smem + L::R_OFF);
  float2_t* table = reinterpret_cast<float2_t*>(smem + L::T_OFF);
  GemmProblem unused = p0;
  const PipeRange R = pipe_range<S::BM>(p0, unused, 0);
  int v = R.t_first;  // position in this XCD's tile sequence
  if (v >= R.t_end) return;  // no tile for this workgroup (uniform)
  int t = R.tile(v);

  const int lane = threadIdx.x & 63;
  // the wave index and group in scalar registers: barriers are only ever
  // skipped by whole wavefronts, and the LDS bases of the loads are uniform
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int group = wave >> 2;
  const int wm = pp_w4_wm(wave), wn = pp_w4_wn(wave);
  const int wr_total = S::GATEUP ? 2 * p0.N : p0.N;
  const int nk = p0.K / KB;          // stages per tile (a multiple of 4)
  const int ng = nk / L::G_STAGES;   // code groups per tile

  // the scale table: (s, -136 s) for every E4M3 byte
  if (threadIdx.x < 256) {
    const float sc = e4m3_to_f32(threadIdx.x);
    table[threadIdx.x] = float2_t{sc, -136.0f * sc};
  }

  // this lane's share of its group's dequantisation: local row rho of the
  // group's half (code slot row crow), columns 16 h .. 16 h + 15 of the stage
  const int gl = (wave & 3) * 64 + lane;
  const int rho = gl >> 1, h = gl & 1;
  const int crow = L::HALF * group + rho;
  const int cswz = pp_w4_cswz(crow);
  const int rrow = S::GATEUP ? (rho >> 6) * BN + (BN / 2) * group + (rho & 63) : crow;
  const int rpos0 = rrow * KB + pl_swz<KB>(rrow, 2 * h) * 8;
  const int rpos1 = rrow * KB + pl_swz<KB>(rrow, 2 * h + 1) * 8;

  f32x16_t acc[NMAT][TM][TN];
  bf16x8_t fa[2][TM], fb[2][NMAT][TN];
  // HALF: a gate_up tile of at most BM/2 rows, run half-height as in the
  // bf16 tile (row half wm takes rows [wm BM/4, (wm+1) BM/4), its first
  // TM/2 row blocks); the dequantisation is a full tile's
  auto read_stage = [&](int slot, int rslot, auto half_c) __attribute__((always_inline)) {
    constexpr bool HALF = decltype(half_c)::value;
    constexpr int TMH = HALF ? TM / 2 : TM, WMH = HALF ? WM / 2 : WM;
    const uint16_t* As = reinterpret_cast<const uint16_t*>(smem + slot * L::A_BYTES);
    const uint16_t* Bs = ring + rslot * (L::RING / 2);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int chunk = s * 2 + (lane >> 5);
#pragma unroll
      for (int i = 0; i < TMH; ++i) {
        const int r = wm * WMH + i * 32 + (lane & 31);
        fa[s][i] = *reinterpret_cast<const bf16x8_t*>(&As[r * KB + pl_swz<KB>(r, chunk) * 8]);
      }
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int r = m * BN + wn * WN + j * 32 + (lane & 31);
          fb[s][m][j] = *reinterpret_cast<const bf16x8_t*>(&Bs[r * KB + pl_swz<KB>(r, chunk) * 8]);
        }
    }
  };
  // Dequantise this group's half of stream stage `ss` (code slot of its
  // group, piece ss % 4 of each row) into ring slot `rslot`.  In a compute
  // phase (mfma set) the stage's 16 MFMAs go around it in a fixed order of
  // issue: the two LDS reads, two MFMAs while they land, the table read, two
  // more, then one piece of the unpacking after each MFMA (two columns at a
  // time, five VALU instructions; a ring write after each eight columns).
  // An MFMA holds the matrix pipe for 32 cycles, longer than a piece takes to
  // issue.
  auto dequant = [&](int ss, int rslot, bool mfma, auto half_c) __attribute__((always_inline)) {
    constexpr bool HALF = decltype(half_c)::value;
    static_assert(2 * NMAT * TM * TN == 16, "16 MFMAs per stage");
    const uint8_t* cs = smem + L::C_OFF + ((ss >> 2) & 1) * L::C_SLOT;
    const uint2_t cw = *reinterpret_cast<const uint2_t*>(
        cs + crow * L::C_ROW + (((ss & 3) ^ cswz) << 4) + 8 * h);
    const uint32_t sb = cs[L::C_BYTES + crow];
    uint16_t* rs = ring + rslot * (L::RING / 2);
#define PPW4_MFMA(lo, hi)                          \
    if (mfma) {                                    \
      __builtin_amdgcn_sched_barrier(0);           \
      pp_mfma_range<S, lo, hi, HALF>(acc, fa, fb); \
      __builtin_amdgcn_sched_barrier(0);           \
    }
    PPW4_MFMA(0, 2)
    const float2_t sc = table[sb];
    PPW4_MFMA(2, 4)
    const uint32_t n0 = cw[0] & 0x0F0F0F0Fu;
    const uint32_t p0 = w4_dequant2(n0, W4_SEL0, W4_SEL1, sc[0], sc[1]);
    PPW4_MFMA(4, 5)
    const uint32_t p1 = w4_dequant2(n0, W4_SEL2, W4_SEL3, sc[0], sc[1]);
    const uint32_t n1 = (cw[0] >> 4) & 0x0F0F0F0Fu;
    PPW4_MFMA(5, 6)
    const uint32_t p2 = w4_dequant2(n1, W4_SEL0, W4_SEL1, sc[0], sc[1]);
    PPW4_MFMA(6, 7)
    const uint32_t p3 = w4_dequant2(n1, W4_SEL2, W4_SEL3, sc[0], sc[1]);
    *reinterpret_cast<u32x4_t*>(rs + rpos0) = u32x4_t{p0, p1, p2, p3};
    PPW4_MFMA(7, 8)
    const uint32_t n2 = cw[1] & 0x0F0F0F0Fu;
    const uint32_t p4 = w4_dequant2(n2, W4_SEL0, W4_SEL1, sc[0], sc[1]);
    PPW4_MFMA(8, 9)
    const uint32_t p5 = w4_dequant2(n2, W4_SEL2, W4_SEL3, sc[0], sc[1]);
    const uint32_t n3 = (cw[1] >> 4) & 0x0F0F0F0Fu;
    PPW4_MFMA(9, 10)
    const uint32_t p6 = w4_dequant2(n3, W4_SEL0, W4_SEL1, sc[0], sc[1]);
    PPW4_MFMA(10, 11)
    const uint32_t p7 = w4_dequant2(n3, W4_SEL2, W4_SEL3, sc[0], sc[1]);
    *reinterpret_cast<u32x4_t*>(rs + rpos1) = u32x4_t{p4, p5, p6, p7};
    PPW4_MFMA(11, 16)
#undef PPW4_MFMA
  };
  auto pp_barrier = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    pl_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  PpW4Tile<S> cur, nxt;
  pp_w4_locate_begin<S>(p0, R.mt0, t, wave, cur);
  pipe_locate_end<S>(p0.K, cur.t);
  // The stream: stage ss of the workgroup's stage stream (ss counts across
  // tiles; every tile has nk stages, a multiple of 4) sits in A slot
  // ss % STAGES and ring slot ss % 2; code group ss / 4 in code slot
  // (ss / 4) % 2.  The prologue loads code group 0, then A stages
  // 0..AHEAD-1.
  pp_w4_issue_c<S>(cur, smem, 0, 0, wave, wr_total);
#pragma unroll
  for (int s0 = 0; s0 < AHEAD; ++s0) pp_w4_issue_a<S>(cur, smem, s0, s0 * KB, wave);
  PL_WAIT_VM_LDS((AHEAD - 1) * L::A_VM);
  pp_barrier();  // code group 0, A stage 0 and the table everywhere
  dequant(0, 0, false, std::false_type{});
  PL_WAIT_LDS();
  pp_barrier();  // stage 0's weights in ring slot 0
  if (group) pp_barrier();
  pipe_store_none<S>(p0);
  int ss = 0;  // stream index of the stage being read
  // Step kt of a tile: read stream stage ss; at a code group's first stage,
  // this group's half of code group cg of tile src (the next group: of this
  // tile, else group 0 of the next one), then A stage k0 of src (AHEAD
  // ahead); wait for this wave's loads of A stage ss+1 (and, with them,
  // every code load issued before it); dequantise stage ss+1 beside this
  // stage's MFMAs.  As in the bf16 tile, the first AHEAD-1 steps of a tile
  // (RELAXED) also let the previous epilogue's S::STORES stores stay in
  // flight (issued after this tile's A stages 0..AHEAD-1 and code group 0,
  // before its code group 1 and A stage AHEAD).
  auto step = [&](int kt, const PpW4Tile<S>& src, int cg, int k0, auto relaxed_c, auto half_c)
                  __attribute__((always_inline)) {
    constexpr int EXTRA = decltype(relaxed_c)::value ? S::STORES : 0;
    read_stage(ss % STAGES, ss & 1, half_c);
    if ((kt & 3) == 0)
      pp_w4_issue_c<S>(src, smem, (ss / L::G_STAGES + 1) & 1, cg, wave, wr_total);
    pp_w4_issue_a<S>(src, smem, (ss + AHEAD) % STAGES, k0, wave);
    if ((kt & 3) == 3)
      PL_WAIT_VM_LDS((AHEAD - 1) * L::A_VM + EXTRA);
    else
      PL_WAIT_VM_LDS((AHEAD - 1) * L::A_VM + L::C_VM + EXTRA);
    pp_barrier();
    dequant(ss + 1, (ss + 1) & 1, true, half_c);  // the next stage, beside this one's MFMAs
    PL_WAIT_LDS();
    pp_barrier();
    ++ss;
  };
  using T0 = std::integral_constant<bool, false>;
  using T1 = std::integral_constant<bool, true>;
  static_assert(AHEAD == L::G_STAGES, "the first AHEAD steps issue code group 1 only");
  for (;;) {
    const bool more = v + R.stride < R.t_end;
    const int t_next = more ? R.tile(v + R.stride) : t;
    // as in the bf16 tile: the next tile's A rows load during the first
    // AHEAD steps (whose stages are all this tile's: nk >= 2 AHEAD), and
    // the last AHEAD steps issue the next tile's first code group and A
    // stages (past the last tile, this tile's again, into free slots)
    if (more) pp_w4_locate_begin<S>(p0, R.mt0, t_next, wave, nxt);
    pipe_zero<S>(acc);
    auto run = [&](auto h) __attribute__((always_inline)) {
#pragma unroll
      for (int kt = 0; kt < AHEAD - 1; ++kt) step(kt, cur, 1, (kt + AHEAD) * KB, T1{}, h);
      step(AHEAD - 1, cur, 1, (2 * AHEAD - 1) * KB, T0{}, h);
      if (more)
        pipe_locate_end<S>(p0.K, nxt.t);
      else
        nxt = cur;
      for (int kt = AHEAD; kt < nk - AHEAD; ++kt)
        step(kt, cur, kt / L::G_STAGES + 1, (kt + AHEAD) * KB, T0{}, h);
#pragma unroll 1
      for (int q = 0; q < AHEAD; ++q) step(nk - AHEAD + q, nxt, 0, q * KB, T0{}, h);
      pipe_store<S, decltype(h)::value>(p0, cur.t, acc, limit, wm, wn);
    };
    // (down keeps full tiles: the half-height copy of its steps spills)
    if (S::GATEUP && cur.t.row_end - cur.t.row0 <= S::BM / 2)
      run(std::integral_constant<bool, S::GATEUP>{});
    else
      run(T0{});
    if (!more) break;
    v += R.stride;
    t = t_next;
    cur = nxt;
  }
  // pairs with group 1's last barrier
  if (group == 0) pp_barrier();
}

// ---------------------------------------------------------------------------
// Persistent weight-streaming variant for short expert segments (decode).
//
// With a few rows per expert every weight byte feeds a few MACs, so the
// projection runs at the rate HBM delivers weights.  HBM3E here gives its
// best rate when each weight row is read in long contiguous pieces (about
// 6.2 TB/s for 512-byte pieces, 5.2 TB/s for the 128-byte pieces of a
// 64-wide K step), so a workgroup owns only 64 weight rows and reads KB*2
// contiguous bytes of each per stage through direct global->LDS loads (1 KB
// per instruction: RPI whole row pieces), STAGES-1 stages in flight.  K needs
// only be a multiple of 32: in a last, partial stage the lanes past K fetch
// the stage's last valid chunk again and the 32-wide substeps past K are
// skipped.
//
// A tile is 16 rows of A (one v_mfma_f32_16x16x32_bf16 row block) by the 64
// weight rows; wavefront w owns weight rows 16w .. 16w+15 and runs every K
// substep for them, so no partial sums cross wavefronts.  In gate_up those
// 16 rows are 8 gate rows and the matching 8 up rows: MFMA columns j and
// j+8 of a lane group hold g and u of one output column, which meet through
// a lane shuffle for the clamped SwiGLU.  Down: 16 output columns per wave.
//
// One workgroup per CU walks a share of its XCD's contiguous range of the
// dense tile list and keeps its loads running across tile boundaries: the
// first stages of the next tile are in flight while the current one is
// stored.  Per-tile lookups (segment offsets, m-tile prefix, gathered row
// ids) are uniform and go through the scalar cache.  Inside an expert the
// m-tiles of one weight tile are adjacent, so when a segment spans several
// m-tiles the repeated weight reads are served by L2.
constexpr int WS_BM = 16;  // A rows per tile
constexpr int WS_NB = 64;  // weight rows per tile (16 per wavefront)

__device__ __forceinline__ int ws_swz(int row, int chunk) {
  // rows are a multiple of 256 bytes long: the 16 rows one ds_read_b128 pass
  // touches must sit in 16 different 16-byte bank groups
  return chunk ^ (row & 15);
}

// One problem's fields, selected between the two problems of the launch.
struct WsProb {
  const uint16_t* A;
  const int32_t* row_index;
  const int32_t* offs;
  const int32_t* mstart;
  const uint16_t* W;
  int64_t w_stride;
  const float* tscale;
  void* out;
  int64_t M;
  int G, N, K, ntiles, mt_total;
};

__device__ __forceinline__ WsProb ws_pick(const GemmProblem& a, const GemmProblem& b, bool second,
                                          int mt_a, int mt_b) {
  WsProb q;
  q.A = second ? b.A : a.A;
  q.row_index = second ? b.row_index : a.row_index;
  q.offs = second ? b.group_offsets : a.group_offsets;
  q.mstart = second ? b.mtile_start : a.mtile_start;
  q.W = second ? b.W : a.W;
  q.w_stride = second ? b.w_stride : a.w_stride;
  q.tscale = second ? b.tscale : a.tscale;
  q.out = second ? b.out : a.out;
  q.M = second ? b.M : a.M;
  q.G = second ? b.G : a.G;
  q.N = second ? b.N : a.N;
  q.K = second ? b.K : a.K;
  q.ntiles = second ? b.ntiles : a.ntiles;
  q.mt_total = second ? mt_b : mt_a;
  return q;
}

// Dense tile t of a problem -> rows [row0, row_end) of group g, columns from
// n0.  Within a group the m-tiles of one n-tile are adjacent.  g comes in as
// the group of an earlier tile of the same problem (a workgroup's tiles only
// move forward, usually within the same group: a short forward scan), or
// negative (binary search).
template <int BN>
__device__ __forceinline__ void ws_locate(const WsProb& P, int t, int64_t& row0, int64_t& row_end,
                                          int& n0, int& g) {
  if (P.offs == nullptr) {
    const int nt = t / P.mt_total, mt = t - nt * P.mt_total;
    g = 0;
    row0 = (int64_t)mt * WS_BM;
    row_end = P.M;
    n0 = nt * BN;
    return;
  }
  // g = last group with mstart[g] * ntiles <= t (its m-tile count is > 0)
  if (g < 0) {
    int lo = 0, hi = P.G - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (ws_sload(P.mstart, mid) * P.ntiles <= t) lo = mid; else hi = mid - 1;
    }
    g = lo;
  } else {
    while (g + 1 < P.G && ws_sload(P.mstart, g + 1) * P.ntiles <= t) ++g;
  }
  const int m_first = ws_sload(P.mstart, g);
  const int mcount = ws_sload(P.mstart, g + 1) - m_first;
  const int local = t - m_first * P.ntiles;
  const int nt = local / mcount, mt = local - nt * mcount;
  row0 = ws_sload(P.offs, g) + (int64_t)mt * WS_BM;
  row_end = ws_sload(P.offs, g + 1);
  n0 = nt * BN;
}

template <bool GATEUP, int KB, int STAGES>
__global__ __launch_bounds__(256, 1) void grouped_wstream_kernel(GemmProblem p0, GemmProblem p1,
                                                                 int has_p1, float limit) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem_dyn[];
  constexpr int BM = WS_BM, NB = WS_NB;
  constexpr int BN = GATEUP ? NB / 2 : NB;  // output columns per tile
  constexpr int ROWS = BM + NB;             // LDS rows per stage
  constexpr int CHUNKS = KB / 8;            // 16-byte chunks per row piece
  constexpr int STAGE = ROWS * KB;          // bf16 elements per stage
  constexpr int RPI = 64 / CHUNKS;          // row pieces per 1 KB load instruction
  constexpr int INSTR = ROWS / RPI;
  constexpr int PER_WAVE = INSTR / 4;
  constexpr int A_INSTR = BM / (4 * RPI);   // instructions of each wave that fill A rows
  constexpr int SUB = KB / 32;              // 32-wide K substeps per stage
  static_assert(INSTR % 4 == 0 && BM % (4 * RPI) == 0 && CHUNKS >= 16, "shape");
  static_assert((STAGES - 2) * PER_WAVE <= 63, "vmcnt range");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  const int mt0 = pipe_mtiles<BM>(p0);
  const int mt1 = has_p1 ? pipe_mtiles<BM>(p1) : 0;
  const int tiles0 = mt0 * p0.ntiles;
  const int total = tiles0 + mt1 * p1.ntiles;
  // each XCD takes a contiguous tile range of equal cost (K stages: the two
  // problems' K may differ), which its workgroups stride
  const int nk0 = (p0.K + KB - 1) / KB, nk1 = (p1.K + KB - 1) / KB;
  const int64_t c0 = (int64_t)tiles0 * nk0;
  const int64_t ctot = c0 + (int64_t)(total - tiles0) * nk1;
  auto first_tile_from = [&](int64_t c) {  // first tile starting at cost >= c
    return c <= c0 ? (int)((c + nk0 - 1) / nk0) : tiles0 + (int)((c - c0 + nk1 - 1) / nk1);
  };
  const int nwg = gridDim.x, b = blockIdx.x;
  const int xcd = b & 7, lid = b >> 3;
  const int nwg_x = (nwg - xcd + 7) >> 3;
  const int t_begin = first_tile_from(ctot * xcd / 8);
  const int t_end = first_tile_from(ctot * (xcd + 1) / 8);
  if (t_begin + lid >= t_end) return;

  // ---- load cursor: tile t_ld, K stage kt_ld, LDS slot slot_ld
  int t_ld = t_begin + lid, kt_ld = 0, slot_ld = 0, nk_ld = 1, K_ld = 0;
  const uint16_t* ld_A = nullptr;
  const uint16_t* ld_W = nullptr;
  uint32_t off[PER_WAVE];
  int g_ld = -1;
  bool sec_ld = false;
  auto setup_ld = [&]() __attribute__((always_inline)) {
    const bool sec = t_ld >= tiles0;
    if (sec != sec_ld) g_ld = -1;
    sec_ld = sec;
    const WsProb P = ws_pick(p0, p1, sec, mt0, mt1);
    int64_t row0, row_end;
    int n0;
    ws_locate<BN>(P, sec ? t_ld - tiles0 : t_ld, row0, row_end, n0, g_ld);
    ld_A = P.A;
    ld_W = P.W + (int64_t)g_ld * P.w_stride;
    nk_ld = (P.K + KB - 1) / KB;
    K_ld = P.K;
    // instruction i of this wave fills stage rows RPI*q .. RPI*q+RPI-1,
    // q = wave + 4i; lane L writes row RPI*q + L/CHUNKS, slot L%CHUNKS, which
    // holds logical chunk ws_swz(row, slot); A rows past the segment and
    // weight rows past N fetch the tile's first row (their products reach
    // only outputs that are never stored)
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int chunk = ws_swz(RPI * (wave + 4 * i) + lane / CHUNKS, lane % CHUNKS);
      if (i < A_INSTR) {
        int64_t src[RPI];
#pragma unroll
        for (int j = 0; j < RPI; ++j) {
          const int64_t gr = row0 + RPI * (wave + 4 * i) + j;
          const int64_t r = gr < row_end ? gr : row0;
          src[j] = P.row_index ? (int64_t)ws_sload(P.row_index, r) : r;
        }
        int64_t mine = src[0];
#pragma unroll
        for (int j = 1; j < RPI; ++j)
          if (lane / CHUNKS == j) mine = src[j];
        off[i] = (uint32_t)(mine * P.K + chunk * 8);
      } else {
        // weight row r of the tile: wave r/16's block; in gate_up its first 8
        // rows are gate rows and the next 8 the matching up rows
        const int r = RPI * (wave + 4 * i) + lane / CHUNKS - BM;
        int n = GATEUP ? n0 + 8 * (r >> 4) + (r & 7) : n0 + r;
        const bool up = GATEUP && (r & 8);
        if (n >= P.N) n = n0;
        off[i] = (uint32_t)((int64_t)(up ? P.N + n : n) * P.K + chunk * 8);
      }
    }
  };
  auto issue_next = [&]() __attribute__((always_inline)) {
    if (t_ld >= t_end) return;
    uint16_t* base = smem_dyn + slot_ld * STAGE;
    const int k0 = kt_ld * KB;
    if (k0 + KB <= K_ld) {
#pragma unroll
      for (int i = 0; i < PER_WAVE; ++i) {
        if (i < A_INSTR)
          lds_direct_16(ld_A + off[i] + k0, base + (wave + 4 * i) * RPI * KB);
        else
          lds_direct_16_stream(ld_W + off[i] + k0, base + (wave + 4 * i) * RPI * KB);
      }
    } else {
      // partial stage: lanes past K fetch the stage's last valid chunk of
      // their row again (same cache line as a valid lane; never read)
      const int last = ((K_ld - k0) >> 3) - 1;
#pragma unroll
      for (int i = 0; i < PER_WAVE; ++i) {
        const int chunk = ws_swz(RPI * (wave + 4 * i) + lane / CHUNKS, lane % CHUNKS);
        const uint32_t o = off[i] + k0 - (uint32_t)(chunk > last ? chunk - last : 0) * 8;
        if (i < A_INSTR)
          lds_direct_16(ld_A + o, base + (wave + 4 * i) * RPI * KB);
        else
          lds_direct_16_stream(ld_W + o, base + (wave + 4 * i) * RPI * KB);
      }
    }
    slot_ld = slot_ld + 1 == STAGES ? 0 : slot_ld + 1;
    if (++kt_ld == nk_ld) {
      kt_ld = 0;
      t_ld += nwg_x;
      if (t_ld < t_end) setup_ld();
    }
  };

  // ---- compute cursor
  int t_cp = t_begin + lid, kt_cp = 0, slot_cp = 0, nk_cp = 1, N_cp = 0, K_cp = 0;
  int64_t row0_cp = 0, row_end_cp = 0;
  int n0_cp = 0;
  void* out_cp = nullptr;
  float ts_cp = 1.0f;  // the tile's group output scale
  int g_cp = -1;
  bool sec_cp = false;
  auto setup_cp = [&]() __attribute__((always_inline)) {
    const bool sec = t_cp >= tiles0;
    if (sec != sec_cp) g_cp = -1;
    sec_cp = sec;
    const WsProb P = ws_pick(p0, p1, sec, mt0, mt1);
    ws_locate<BN>(P, sec ? t_cp - tiles0 : t_cp, row0_cp, row_end_cp, n0_cp, g_cp);
    nk_cp = (P.K + KB - 1) / KB;
    K_cp = P.K;
    N_cp = P.N;
    out_cp = P.out;
    ts_cp = P.tscale ? ws_sloadf(P.tscale, g_cp) : 1.0f;
  };

  // element (reg r, lane l) of the wave's accumulator: row 4(l/16) + r of
  // the tile, weight row 16*wave + l%16
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  const int fr = lane & 15;       // fragment row (A) / weight row within the wave's block
  auto store = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t row = row0_cp + 4 * (lane >> 4) + r;
      const float v = acc[r] * ts_cp;
      if (GATEUP) {
        const float u = __shfl_xor(v, 8, 64);  // lanes j, j+8: g and u of one column
        const int col = n0_cp + 8 * wave + (fr & 7);
        if (fr < 8 && row < row_end_cp && col < N_cp)
          static_cast<uint16_t*>(out_cp)[row * N_cp + col] =
              (uint16_t)f32_to_bf16_bits(swiglu_clamped(v, u, limit));
      } else {
        const int col = n0_cp + 16 * wave + fr;
        if (row < row_end_cp && col < N_cp) static_cast<float*>(out_cp)[row * N_cp + col] = v;
      }
    }
  };
  auto substep = [&](const uint16_t* As, const uint16_t* Bs, int ks) __attribute__((always_inline)) {
    const int chunk = ks * 4 + (lane >> 4);
    const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(&As[fr * KB + ws_swz(fr, chunk) * 8]);
    const int br = 16 * wave + fr;
    const bf16x8_t bv = *reinterpret_cast<const bf16x8_t*>(&Bs[br * KB + ws_swz(BM + br, chunk) * 8]);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bv, acc, 0, 0, 0);
  };

  setup_ld();
  setup_cp();
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s) issue_next();

  while (true) {
    // own loads of this stage landed (at most STAGES-2 newer stages in
    // flight while the loader still has work), own LDS reads done; after
    // the barrier the stage is complete everywhere and the slot the next
    // loads overwrite (read in the previous step) is free
    if (t_ld < t_end)
      PL_WAIT_VM_LDS((STAGES - 2) * PER_WAVE);
    else
      PL_WAIT_VM_LDS(0);
    pl_barrier();
    issue_next();
    const uint16_t* As = smem_dyn + slot_cp * STAGE;
    const uint16_t* Bs = As + BM * KB;
    const int sub_valid = (K_cp - kt_cp * KB) >> 5;  // 32-wide substeps left in K
    if (sub_valid >= SUB) {
#pragma unroll
      for (int ks = 0; ks < SUB; ++ks) substep(As, Bs, ks);
    } else {
      for (int ks = 0; ks < sub_valid; ++ks) substep(As, Bs, ks);
    }
    slot_cp = slot_cp + 1 == STAGES ? 0 : slot_cp + 1;
    if (++kt_cp == nk_cp) {
      store();
      t_cp += nwg_x;
      if (t_cp >= t_end) break;
      kt_cp = 0;
      setup_cp();
      acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  }
}

// ---------------------------------------------------------------------------
// Weight streaming with W4A16 weights (decode; the grouped W4A16 expert GEMM
// of "Module glm5next_mlp", in this library's format: 4-bit codes u of value
// u - 8, packed along K in 4-byte words of 8 columns whose byte j holds
// columns j and j + 4 in its low and high nibble, one E4M3 scale byte per
// weight row and 128 columns, stored group-major, and one fp32 tensor scale
// per expert, applied to the accumulators before the store).
//
// At a quarter of the bf16 size per weight, a 64-row weight tile would take
// no more LDS per stage than the 16 gathered A rows and halve the weight bytes
// in flight.  So a tile here is 16 A rows by NB = 16 * NBLK * NW weight rows:
// each of the NW wavefronts owns NBLK blocks of 16 weight rows, which share
// its A fragments; a stage covers KB columns of K (whole 128-column groups).
// Unlike the bf16 kernel this one has real per-weight ALU work (unpacking
// the codes), so it runs two wavefronts per SIMD: one's unpacking overlaps
// the other's MFMAs.  A rows past the segment are not fetched (a lane-0 load
// keeps each wavefront's count of loads per stage fixed); their products
// reach only rows that are never stored.
//
// Per stage and weight block a lane reads one 16-byte piece of codes: lane
// group q (lane / 16) takes piece 4s + q of the row's stage span, whose four
// dwords feed substeps 4s .. 4s+3, and its A fragment in substep 4s + t is
// columns 32 (4s + q) + 8t .. +7 of its row; a 128-column group is thus four
// substeps.  A code dword becomes eight bf16 values 128 + u exactly (bits
// 0x4300 | u: one mask per nibble half, then a byte permute per pair); the
// MFMA sums
// x (128 + u) over the group, one more MFMA against ones sums x (shared by
// the blocks), and scale (P - 136 X) = scale * sum x (u - 8) goes into the
// fp32 accumulator.  K must be a multiple of 128; a last stage with fewer
// groups than KB / 128 fetches an earlier group again in place of the
// missing ones and computes only its own.

// the launched shape: 256 weight rows by 256 columns a stage, eight
// wavefronts, three stages
constexpr int W4_NBLK = 2, W4_KB = 256, W4_NW = 8, W4_STAGES = 3;

template <int NBLK, int KB, int NW>
struct W4Shape {
  static constexpr int NB = 16 * NBLK * NW;        // weight rows per tile
  static constexpr int A_BYTES = WS_BM * KB * 2;   // 16 rows of bf16
  static constexpr int W_ROW = KB / 2;             // code bytes per weight row and stage
  static constexpr int W_BYTES = NB * W_ROW;
  static constexpr int S_WAVE = NBLK * KB / 8;     // scale bytes per wavefront and stage
  static constexpr int STAGE = A_BYTES + W_BYTES + NW * S_WAVE;
  static constexpr int A_CH = KB / 8;              // 16-byte chunks per A row
  static constexpr int A_RPI = 64 / A_CH;          // A rows per 1 KB instruction
  static constexpr int A_PW = WS_BM / (NW * A_RPI);  // A instructions per wavefront
  static constexpr int W_CH = KB / 32;             // 16-byte pieces per weight row
  static constexpr int W_RPI = 64 / W_CH;          // weight rows per instruction
  static constexpr int W_PW = NB / (NW * W_RPI);   // weight instructions per wavefront
  static constexpr int S_LANES = S_WAVE / 16;      // lanes that fetch the scales
  static constexpr int PER_WAVE = A_PW + W_PW + 1;
  static constexpr int GROUPS = KB / 128;          // scale groups per stage
  // a 16-byte piece of scale bytes covers 16 rows: one block (down) or the
  // gate or up halves of two blocks (gate_up)
  static_assert(NBLK % 2 == 0, "whole 16-byte scale pieces");
  static_assert(KB % 128 == 0 && KB <= 512 && A_PW >= 1 && A_PW * NW * A_RPI == WS_BM &&
                W_PW >= 1 && W_PW * NW * W_RPI == NB && S_LANES >= 1 && S_LANES <= 64,
                "W4 shape");
};

// weight row r's 16-byte piece c sits in slot w4_swz: the 16 rows one
// ds_read_b128 pass touches land in 16 different 16-byte bank groups
template <int W_CH>
__device__ __forceinline__ int w4_swz(int r, int c) {
  return c ^ ((r / (16 / W_CH)) & (W_CH - 1));
}

__device__ __forceinline__ bf16x8_t w4_codes_to_bf16(uint32_t d) {
  // byte j of d holds columns j (low nibble) and j + 4 (high nibble): the
  // masks give the bytes u of columns 0..3 and 4..7; each permute takes two
  // of them as the low bytes of a pair and 0x43 as the high bytes
  const uint32_t lo = d & 0x0F0F0F0Fu, hi = (d >> 4) & 0x0F0F0F0Fu;
  uint32_t o[4];
  o[0] = __builtin_amdgcn_perm(0x43434343u, lo, 0x04010400u);  // columns 0, 1
  o[1] = __builtin_amdgcn_perm(0x43434343u, lo, 0x04030402u);  // columns 2, 3
  o[2] = __builtin_amdgcn_perm(0x43434343u, hi, 0x04010400u);  // columns 4, 5
  o[3] = __builtin_amdgcn_perm(0x43434343u, hi, 0x04030402u);  // columns 6, 7
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t v = {o[0], o[1], o[2], o[3]};
  return __builtin_bit_cast(bf16x8_t, v);
}

template <bool GATEUP, int NBLK, int KB, int NW, int STAGES>
__global__ __launch_bounds__(NW * 64, 1) void grouped_wstream_w4_kernel(GemmProblem p0,
                                                                       float limit) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem_dyn[];
  using S = W4Shape<NBLK, KB, NW>;
  constexpr int BM = WS_BM, NB = S::NB;
  constexpr int BN = GATEUP ? NB / 2 : NB;  // output columns per tile
  static_assert((STAGES - 2) * S::PER_WAVE <= 63 && STAGES * S::STAGE <= 160 * 1024, "stages");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint8_t* const smem = reinterpret_cast<uint8_t*>(smem_dyn);

  const int mt0 = pipe_mtiles<BM>(p0);
  const int total = mt0 * p0.ntiles;
  const int nk = (p0.K + KB - 1) / KB;
  const int nwg = gridDim.x, b = blockIdx.x;
  const int xcd = b & 7, lid = b >> 3;
  const int nwg_x = (nwg - xcd + 7) >> 3;
  const int t_begin = (int)((int64_t)total * xcd / 8);
  const int t_end = (int)((int64_t)total * (xcd + 1) / 8);
  if (t_begin + lid >= t_end) return;
  const WsProb P = ws_pick(p0, p0, false, mt0, mt0);
  const int K = P.K, N = P.N;
  const int groups = K / 128;
  const int rs = GATEUP ? 2 * N : N;  // scale entries per group

  // ---- load cursor
  int t_ld = t_begin + lid, kt_ld = 0, slot_ld = 0, g_ld = -1, rows_ld = 0;
  const uint16_t* ld_A = P.A;
  const uint8_t* ld_W = nullptr;
  const uint8_t* ld_S = nullptr;
  uint32_t offA[S::A_PW], offW[S::W_PW], offS = 0;
  auto setup_ld = [&]() __attribute__((always_inline)) {
    int64_t row0, row_end;
    int n0;
    ws_locate<BN>(P, t_ld, row0, row_end, n0, g_ld);
    rows_ld = (int)(row_end - row0);
    ld_W = reinterpret_cast<const uint8_t*>(P.W) + (int64_t)g_ld * P.w_stride * 2;
    ld_S = p0.S + (int64_t)g_ld * p0.s_stride;
    // A: instruction i of wave w fills rows A_RPI q .. A_RPI q + A_RPI - 1,
    // q = w + NW i; lane L writes row A_RPI q + L / A_CH, slot L % A_CH,
    // which holds logical chunk slot ^ (row & 15).  Rows past the segment
    // point at the tile's first row (only lane 0 fetches there).
#pragma unroll
    for (int i = 0; i < S::A_PW; ++i) {
      // the instruction's A_RPI row ids are uniform: scalar loads, then each
      // lane takes its own
      int64_t mine = 0;
#pragma unroll
      for (int j = 0; j < S::A_RPI; ++j) {
        const int64_t gr = row0 + S::A_RPI * (wave + NW * i) + j;
        const int64_t rr = gr < row_end ? gr : row0;
        const int64_t src = P.row_index ? (int64_t)ws_sload(P.row_index, rr) : rr;
        if (lane / S::A_CH == j) mine = src;
      }
      const int r = S::A_RPI * (wave + NW * i) + lane / S::A_CH;
      offA[i] = (uint32_t)(mine * K + ((lane % S::A_CH) ^ (r & 15)) * 8);
    }
    // W: instruction i of wave w fills weight rows W_RPI q .. , q = w + NW i;
    // lane L writes row W_RPI q + L / W_CH, slot L % W_CH.  Block b (wave
    // b / NBLK's block b % NBLK) holds tile rows 16 b .. 16 b + 15: in gate_up
    // 8 gate rows and the matching 8 up rows.  Rows past N fetch row n0.
#pragma unroll
    for (int i = 0; i < S::W_PW; ++i) {
      const int r = S::W_RPI * (wave + NW * i) + lane / S::W_CH;
      int n = GATEUP ? n0 + 8 * (r >> 4) + (r & 7) : n0 + r;
      const bool up = GATEUP && (r & 8);
      if (n >= N) n = n0;
      const int c = w4_swz<S::W_CH>(r, lane % S::W_CH);
      offW[i] = (uint32_t)((int64_t)(up ? N + n : n) * (K / 2) + c * 16);
    }
    // E4M3 scale bytes of the wave's rows, per group of the stage: in
    // gate_up 8 NBLK gate rows then the same up rows, in down 16 NBLK rows,
    // in 16-byte pieces (NBLK per group); lane l < S_LANES fetches piece
    // l % NBLK of stage group l / NBLK; offS is the piece's byte offset
    // within a group
    if (lane < S::S_LANES) {
      const int pi = lane % NBLK;
      int n;
      bool up = false;
      if (GATEUP) {
        up = pi >= NBLK / 2;
        n = n0 + 8 * NBLK * wave + 16 * (up ? pi - NBLK / 2 : pi);
      } else {
        n = n0 + 16 * NBLK * wave + 16 * pi;
      }
      if (n >= N) n = n0;
      offS = (uint32_t)(up ? N + n : n);
    }
  };
  auto issue_next = [&]() __attribute__((always_inline)) {
    if (t_ld >= t_end) return;
    uint8_t* base = smem + slot_ld * S::STAGE;
    const int k0 = kt_ld * KB;
    const int gv = min(S::GROUPS, groups - k0 / 128);  // groups of K in this stage
#pragma unroll
    for (int i = 0; i < S::A_PW; ++i) {
      // chunks past K fetch the chunk 128 columns (or more) back: never read
      const int r = S::A_RPI * (wave + NW * i) + lane / S::A_CH;
      const int chunk = (lane % S::A_CH) ^ (r & 15);
      const int back = chunk / 16 >= gv ? (chunk / 16 - gv + 1) * 128 : 0;
      const uint32_t o = offA[i] + (uint32_t)k0 - (uint32_t)back;  // >= 0: back <= 8 chunk
      if (r < rows_ld || lane == 0)
        lds_direct_16(ld_A + o, reinterpret_cast<uint16_t*>(base + (wave + NW * i) * 1024));
    }
#pragma unroll
    for (int i = 0; i < S::W_PW; ++i) {
      const int r = S::W_RPI * (wave + NW * i) + lane / S::W_CH;
      const int c = w4_swz<S::W_CH>(r, lane % S::W_CH);
      const int back = c / 4 >= gv ? (c / 4 - gv + 1) * 64 : 0;
      const uint32_t o = offW[i] + (uint32_t)(k0 / 2) - (uint32_t)back;  // >= 0: back <= 16 c
      lds_direct_16_stream(ld_W + o,
                           reinterpret_cast<uint16_t*>(base + S::A_BYTES + (wave + NW * i) * 1024));
    }
    if (lane < S::S_LANES) {
      // K group of the piece; groups past K fetch the stage's last one again
      const int gk = k0 / 128 + min(lane / NBLK, gv - 1);
      lds_direct_16_stream(ld_S + (offS + (uint32_t)gk * (uint32_t)rs),
                           reinterpret_cast<uint16_t*>(base + S::A_BYTES + S::W_BYTES +
                                                       wave * S::S_WAVE));
    }
    slot_ld = slot_ld + 1 == STAGES ? 0 : slot_ld + 1;
    if (++kt_ld == nk) {
      kt_ld = 0;
      t_ld += nwg_x;
      if (t_ld < t_end) setup_ld();
    }
  };

  // ---- compute cursor
  int t_cp = t_begin + lid, kt_cp = 0, slot_cp = 0, g_cp = -1, n0_cp = 0;
  int64_t row0_cp = 0, row_end_cp = 0;
  float ts_cp = 1.0f;  // the expert's tensor scale
  auto setup_cp = [&]() __attribute__((always_inline)) {
    ws_locate<BN>(P, t_cp, row0_cp, row_end_cp, n0_cp, g_cp);
    ts_cp = P.tscale ? ws_sloadf(P.tscale, g_cp) : 1.0f;
  };

  // element (reg r, lane l) of block j's accumulator: row 4(l/16) + r of the
  // tile, weight row 16 (NBLK wave + j) + l%16
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
  f32x4_t acc[NBLK];
#pragma unroll
  for (int j = 0; j < NBLK; ++j) acc[j] = zero;
  const int fr = lane & 15, q = lane >> 4;
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, u32x4_t{0x3F803F80u, 0x3F803F80u,
                                                             0x3F803F80u, 0x3F803F80u});
  auto store = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NBLK; ++j) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = row0_cp + 4 * q + r;
        const float v = acc[j][r] * ts_cp;
        if (GATEUP) {
          const float u = __shfl_xor(v, 8, 64);  // lanes i, i+8: g and u of one column
          const int col = n0_cp + 8 * (NBLK * wave + j) + (fr & 7);
          if (fr < 8 && row < row_end_cp && col < N)
            static_cast<uint16_t*>(P.out)[row * N + col] =
                (uint16_t)f32_to_bf16_bits(swiglu_clamped(v, u, limit));
        } else {
          const int col = n0_cp + 16 * (NBLK * wave + j) + fr;
          if (row < row_end_cp && col < N) static_cast<float*>(P.out)[row * N + col] = v;
        }
      }
    }
  };
  // one 128-column group s of the stage at base: four substeps (the first
  // MFMA of each sum starts from zero), then the scaled fold
  auto group = [&](const uint8_t* base, int s) __attribute__((always_inline)) {
    const uint16_t* As = reinterpret_cast<const uint16_t*>(base);
    const uint8_t* Ws = base + S::A_BYTES;
    const uint8_t* Ss = base + S::A_BYTES + S::W_BYTES + wave * S::S_WAVE + 16 * NBLK * s;
    u32x4_t codes[NBLK];
#pragma unroll
    for (int j = 0; j < NBLK; ++j) {
      const int br = 16 * (NBLK * wave + j) + fr;
      codes[j] = *reinterpret_cast<const u32x4_t*>(
          &Ws[br * S::W_ROW + w4_swz<S::W_CH>(br, 4 * s + q) * 16]);
    }
    f32x4_t accP[NBLK], accX;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int chunk = 16 * s + 4 * q + t;
      const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(&As[fr * KB + (chunk ^ fr) * 8]);
#pragma unroll
      for (int j = 0; j < NBLK; ++j)
        accP[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, w4_codes_to_bf16(codes[j][t]),
                                                          t == 0 ? zero : accP[j], 0, 0, 0);
      accX = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, ones, t == 0 ? zero : accX, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < NBLK; ++j) {
      const int so = GATEUP ? (fr < 8 ? 0 : 8 * NBLK) + 8 * j + (fr & 7) : 16 * j + fr;
      const float sc = e4m3_to_f32(Ss[so]);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[j][r] = fmaf(sc, fmaf(-136.0f, accX[r], accP[j][r]), acc[j][r]);
    }
  };

  setup_ld();
  setup_cp();
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s) issue_next();

  while (true) {
    // as in the bf16 kernel: own loads of this stage landed, own LDS reads
    // done, then the barrier
    if (t_ld < t_end)
      PL_WAIT_VM_LDS((STAGES - 2) * S::PER_WAVE);
    else
      PL_WAIT_VM_LDS(0);
    pl_barrier();
    issue_next();
    const uint8_t* base = smem + slot_cp * S::STAGE;
    const int gv = groups - kt_cp * S::GROUPS;  // groups of K left
    if (gv >= S::GROUPS) {
#pragma unroll
      for (int s = 0; s < S::GROUPS; ++s) group(base, s);
    } else {
      for (int s = 0; s < gv; ++s) group(base, s);
    }
    slot_cp = slot_cp + 1 == STAGES ? 0 : slot_cp + 1;
    if (++kt_cp == nk) {
      store();
      t_cp += nwg_x;
      if (t_cp >= t_end) break;
      kt_cp = 0;
      setup_cp();
#pragma unroll
      for (int j = 0; j < NBLK; ++j) acc[j] = zero;
    }
  }
}

int device_cu_count() {
  static int cached = 0;  // per process: one device model in a run
  if (cached == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      cached = n;
    else
      cached = 256;
  }
  return cached;
}

template <int BM, int BN, bool GATEUP, int KB, int STAGES, int WAVES_M, int NW, bool PP,
          bool PACKED, bool HBLK>
hipError_t launch_pipe(const GemmProblem& a, const GemmProblem* b, float limit,
                       hipStream_t stream) {
  using S = PipeShape<BM, BN, GATEUP, KB, NW, WAVES_M, PACKED, HBLK>;
  const size_t lds = (size_t)STAGES * S::STAGE * sizeof(uint16_t);
  static_assert((size_t)STAGES * S::STAGE * 2 <= 160 * 1024, "LDS");
  void (*kern)(GemmProblem, GemmProblem, int, float);
  if constexpr (PP)
    kern = grouped_pp_kernel<S, STAGES>;
  else
    kern = grouped_pipe_kernel<S, STAGES>;
  static bool attr_set = false;  // raise the dynamic LDS limit once per process
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const GemmProblem pb = b ? *b : a;
  const int grid = device_cu_count();  // one resident workgroup per CU
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NW * 64), lds, stream, a, pb, b ? 1 : 0, limit);
  return hipGetLastError();
}

template <bool GATEUP>
hipError_t launch_pp_w4(const GemmProblem& a, float limit, hipStream_t stream) {
  using S = PipeShape<256, GATEUP ? 128 : 256, GATEUP, 32, 8, 2>;
  const size_t lds = PpW4Layout<S>::BYTES;
  auto kern = grouped_pp_w4_kernel<S>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(kern, dim3(device_cu_count()), dim3(S::NW * 64), lds, stream, a, limit);
  return hipGetLastError();
}

template <bool GATEUP, int KB, int STAGES>
hipError_t launch_wstream(const GemmProblem& a, const GemmProblem* b, float limit,
                          hipStream_t stream, int max_wgs) {
  const size_t lds = (size_t)STAGES * (WS_BM + WS_NB) * KB * sizeof(uint16_t);
  static_assert((size_t)STAGES * (WS_BM + WS_NB) * KB * 2 <= 160 * 1024, "LDS");
  auto kern = grouped_wstream_kernel<GATEUP, KB, STAGES>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const GemmProblem pb = b ? *b : a;
  // one resident workgroup per CU, or fewer to leave CUs to concurrent work
  const int grid = max_wgs > 0 ? std::min(max_wgs, device_cu_count()) : device_cu_count();
  hipLaunchKernelGGL(kern, dim3(grid), dim3(256), lds, stream, a, pb, b ? 1 : 0, limit);
  return hipGetLastError();
}

template <bool GATEUP, int NBLK, int KB, int NW, int STAGES>
hipError_t launch_wstream_w4(const GemmProblem& a, float limit, hipStream_t stream, int max_wgs) {
  const size_t lds = (size_t)STAGES * W4Shape<NBLK, KB, NW>::STAGE;
  auto kern = grouped_wstream_w4_kernel<GATEUP, NBLK, KB, NW, STAGES>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int grid = max_wgs > 0 ? std::min(max_wgs, device_cu_count()) : device_cu_count();
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NW * 64), lds, stream, a, limit);
  return hipGetLastError();
}

// Tile-blocked copy of expert weights (launch_pack_experts): one workgroup
// of 256 threads per block (group, tile b, K stage s); thread r copies tile
// row r's 32 values (64 bytes, four 16-byte loads and stores).
template <bool GATEUP>
__global__ __launch_bounds__(256) void pack_experts_kernel(const uint16_t* __restrict__ w,
                                                           uint16_t* __restrict__ packed, int N,
                                                           int K, int ntiles) {
  const int nk = K / 32;
  const int64_t blk = blockIdx.x;  // (g * ntiles + b) * nk + s
  const int s = (int)(blk % nk);
  const int64_t gb = blk / nk;
  const int b = (int)(gb % ntiles);
  const int64_t g = gb / ntiles;
  const int r = threadIdx.x;
  int n;
  bool up = false;
  if (GATEUP) {
    up = r >= 128;
    n = 128 * b + (r & 127);
  } else {
    n = 256 * b + r;
  }
  const int64_t rows = GATEUP ? 2 * (int64_t)N : N;
  uint4* dst = reinterpret_cast<uint4*>(packed + (blk * 256 + r) * 32);
  if (n < N) {
    const uint4* src = reinterpret_cast<const uint4*>(
        w + (g * rows + (up ? N + n : n)) * (int64_t)K + (int64_t)s * 32);
#pragma unroll
    for (int q = 0; q < 4; ++q) dst[q] = src[q];
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) dst[q] = make_uint4(0u, 0u, 0u, 0u);
  }
}

// m-tile prefix of up to two tile heights over one set of group offsets.
__global__ __launch_bounds__(1024) void gemm_schedule_kernel(const int32_t* __restrict__ offsets,
                                                             int G, int bm0, int bm1,
                                                             int32_t* __restrict__ start0,
                                                             int32_t* __restrict__ start1) {
  __shared__ int32_t wsum[2][16];
  const int g = threadIdx.x, lane = g & 63, wave = g >> 6;
  int32_t n = (g < G) ? offsets[g + 1] - offsets[g] : 0;
  int32_t v[2] = {(n + bm0 - 1) / bm0, (n + bm1 - 1) / bm1};
  int32_t incl[2] = {v[0], v[1]};
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      int32_t o = __shfl_up(incl[q], off, 64);
      if (lane >= off) incl[q] += o;
    }
  }
  if (lane == 63) { wsum[0][wave] = incl[0]; wsum[1][wave] = incl[1]; }
  __syncthreads();
  int32_t before[2] = {0, 0};
  for (int w = 0; w < wave; ++w) { before[0] += wsum[0][w]; before[1] += wsum[1][w]; }
  if (g < G) {
    start0[g] = before[0] + incl[0] - v[0];
    if (start1) start1[g] = before[1] + incl[1] - v[1];
  }
  if (g == G - 1) {
    start0[G] = before[0] + incl[0];
    if (start1) start1[G] = before[1] + incl[1];
  }
}

template <int BM, int BN, int WM_, int WN_>
hipError_t launch_pair(const GemmProblem& a, const GemmProblem* b, float limit, bool gateup,
                       hipStream_t stream) {
  const int tiles0 = a.max_mtiles * a.ntiles;
  const int tiles1 = b ? b->max_mtiles * b->ntiles : 0;
  const int total = tiles0 + tiles1;
  if (total == 0) return hipSuccess;
  GemmProblem pb = b ? *b : a;
  dim3 grid(total), block(WM_ * WN_ * 64);
  if (gateup)
    hipLaunchKernelGGL((grouped_gemm_kernel<BM, BN, WM_, WN_, true>), grid, block, 0, stream, a,
                       pb, tiles0, limit);
  else
    hipLaunchKernelGGL((grouped_gemm_kernel<BM, BN, WM_, WN_, false>), grid, block, 0, stream, a,
                       pb, tiles0, limit);
  return hipGetLastError();
}

}  // namespace

int gemm_cu_count() { return device_cu_count(); }

int gemm_tile_m(GemmVariant v) {
  switch (v) {
    case GemmVariant::kTile32: return 32;
    case GemmVariant::kTile128: return 128;
    case GemmVariant::kPipe256W8: return 256;
    case GemmVariant::kPingPong: return 256;
    case GemmVariant::kWStream: return WS_BM;
  }
  return 128;
}
int gemm_tile_n(GemmVariant v, bool gateup) {
  if (v == GemmVariant::kWStream) return gateup ? WS_NB / 2 : WS_NB;
  if (v == GemmVariant::kPipe256W8 || v == GemmVariant::kPingPong)
    return gateup ? 128 : 256;
  return 128;
}

int gemm_w4_tile_n(bool gateup) { return gateup ? 8 * W4_NBLK * W4_NW : 16 * W4_NBLK * W4_NW; }

int64_t pack_experts_elems(int G, int N, int K, bool gateup) {
  const int64_t tiles = gateup ? (N + 127) / 128 : (N + 255) / 256;
  return (int64_t)G * tiles * 256 * K;
}

hipError_t launch_pack_experts(const uint16_t* w, uint16_t* packed, int G, int N, int K,
                               bool gateup, hipStream_t stream) {
  const int ntiles = gateup ? (N + 127) / 128 : (N + 255) / 256;
  const int64_t blocks = (int64_t)G * ntiles * (K / 32);
  if (blocks == 0) return hipSuccess;
  if (gateup)
    hipLaunchKernelGGL(pack_experts_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, w,
                       packed, N, K, ntiles);
  else
    hipLaunchKernelGGL(pack_experts_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, w,
                       packed, N, K, ntiles);
  return hipGetLastError();
}

hipError_t launch_gemm_schedule(const int32_t* group_offsets, int G, int bm0, int bm1,
                                int32_t* start0, int32_t* start1, hipStream_t stream) {
  hipLaunchKernelGGL(gemm_schedule_kernel, dim3(1), dim3(1024), 0, stream, group_offsets, G, bm0,
                     bm1, start0, start1);
  return hipGetLastError();
}

// The 256-row tiles over weights in rows of K or tile-blocked (PACKED), h
// in rows or stage-blocked (HBLK).
template <bool PACKED, bool HBLK>
hipError_t launch_pipe_layout(GemmVariant v, bool gateup, const GemmProblem& a,
                              const GemmProblem* b, float limit, hipStream_t stream) {
  // ping-pong: eight wavefronts taking turns on each SIMD; its cross-tile
  // stage stream needs at least 2 (STAGES-1) = 8 stages per tile, so
  // shorter K takes the interleaved schedule of the same tile (eight
  // wavefronts, two per SIMD)
  const bool pp = v == GemmVariant::kPingPong && a.K >= 8 * 32 && (b == nullptr || b->K >= 8 * 32);
  if (pp) {
    if (gateup) return launch_pipe<256, 128, true, 32, 5, 2, 8, true, PACKED, HBLK>(a, b, limit, stream);
    return launch_pipe<256, 256, false, 32, 5, 2, 8, true, PACKED, HBLK>(a, b, limit, stream);
  }
  if (gateup) return launch_pipe<256, 128, true, 32, 5, 2, 8, false, PACKED, HBLK>(a, b, limit, stream);
  return launch_pipe<256, 256, false, 32, 5, 2, 8, false, PACKED, HBLK>(a, b, limit, stream);
}

hipError_t launch_grouped_gemm(GemmVariant v, bool gateup, const GemmProblem& a,
                               const GemmProblem* b, float limit, hipStream_t stream,
                               int max_wgs) {
  if (a.S != nullptr) {  // W4A16 weights: one problem per launch
    if (b != nullptr || a.K % 128 != 0 || a.packed || a.hblk) return hipErrorInvalidValue;
    if (v == GemmVariant::kPingPong) {  // long segments: the ping-pong tile
      if (a.K < 256 || a.N % 32 != 0) return hipErrorInvalidValue;
      if (gateup) return launch_pp_w4<true>(a, limit, stream);
      return launch_pp_w4<false>(a, limit, stream);
    }
    if (v != GemmVariant::kWStream) return hipErrorInvalidValue;
    if (gateup)
      return launch_wstream_w4<true, W4_NBLK, W4_KB, W4_NW, W4_STAGES>(a, limit, stream, max_wgs);
    return launch_wstream_w4<false, W4_NBLK, W4_KB, W4_NW, W4_STAGES>(a, limit, stream, max_wgs);
  }
  // the blocked weight and h layouts are read by the 256-row tiles only,
  // and the problems of one launch share their layouts
  if (b != nullptr && (b->packed != a.packed || b->hblk != a.hblk)) return hipErrorInvalidValue;
  if ((a.packed || a.hblk) && v != GemmVariant::kPingPong && v != GemmVariant::kPipe256W8)
    return hipErrorInvalidValue;
  if (a.packed && a.hblk) return launch_pipe_layout<true, true>(v, gateup, a, b, limit, stream);
  if (a.packed) return launch_pipe_layout<true, false>(v, gateup, a, b, limit, stream);
  if (a.hblk) return launch_pipe_layout<false, true>(v, gateup, a, b, limit, stream);
  if (v == GemmVariant::kTile32) return launch_pair<32, 128, 1, 4>(a, b, limit, gateup, stream);
  if (v == GemmVariant::kWStream) {  // 512-byte row pieces, four stages
    if (gateup) return launch_wstream<true, 256, 4>(a, b, limit, stream, max_wgs);
    return launch_wstream<false, 256, 4>(a, b, limit, stream, max_wgs);
  }
  if (v == GemmVariant::kPipe256W8 || v == GemmVariant::kPingPong)
    return launch_pipe_layout<false, false>(v, gateup, a, b, limit, stream);
  return launch_pair<128, 128, 2, 2>(a, b, limit, gateup, stream);
}
