// Host-side launchers of the gfx950 kernels (one translation unit each).
// Every launcher only enqueues on `stream` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define MOE_MAX_EXPERTS_DEV 1024
#define MOE_MAX_TOP_K_DEV 16
// bytes of the fixed device scratch of moe_forward_noalloc (noalloc.hip)
#define MOE_NOALLOC_SCRATCH_BYTES_DEV ((size_t)64 << 20)

// One grouped GEMM problem: rows of A (optionally gathered through
// row_index) grouped by device offsets, each group against its own weight.
struct GemmProblem {
  const uint16_t* A;              // [rows_a, K] bf16, K contiguous
  const int32_t* row_index;       // [M] source row of each GEMM row, or nullptr
  const int32_t* group_offsets;   // [G+1] device row offsets, or nullptr: one group of M rows
  const int32_t* mtile_start;     // [G+1] device m-tile prefix (with group_offsets)
  const uint16_t* W;              // [G, WR, K] bf16; gate_up: WR = 2N, down: WR = N
                                  // (W4A16: [G, WR, K/2] bytes of 4-bit codes)
  int64_t w_stride;               // uint16 elements between groups of W
  const uint8_t* S;               // W4A16 only: [G, K/128, WR] E4M3 scales; nullptr = bf16 W
  int64_t s_stride;               // bytes between groups of S
  const float* tscale;            // [G] fp32 scale of each group's outputs (the W4A16
                                  // tensor scales, applied to the fp32 accumulators
                                  // before the epilogue), or nullptr = 1
  void* out;                      // [M, N]: bf16 h (gate_up) or fp32 y (down)
  int64_t M;                      // total rows
  int32_t G;                      // groups
  int32_t N;                      // output columns
  int32_t K;                      // reduction length
  int32_t ntiles;                 // ceil(N / BN) (BN of the variant and projection)
  int32_t max_mtiles;             // host bound: ceil(M / BM) + G (or ceil(M / BM) for one group)
  int32_t packed;                 // 1: W in the tile-blocked layout of launch_pack_experts
                                  // (256-row tiles only; w_stride its padded expert size)
  int32_t hblk;                   // 1 (256-row tiles only): gate_up writes `out`, down reads
                                  // A, stage-blocked within each 256-row tile: the tile's
                                  // rows [r0, r0 + n) keep their row-major footprint, with
                                  // columns [32 s, 32 s + 32) of row r0 + r at element
                                  // r0 * K + (s * n + r) * 32 (K: h's width)
};

// Tile variants of the grouped GEMM: persistent weight streaming in long
// row pieces (short expert segments; K a multiple of 32), LDS-staged 32-row
// and 128-row tiles, and pipelined 256-row tiles with direct buffer->LDS
// loads (long segments), eight wavefronts either interleaved or taking turns
// on each SIMD (ping-pong).
enum class GemmVariant { kTile32, kTile128, kWStream, kPipe256W8, kPingPong };
int gemm_tile_m(GemmVariant v);
int gemm_tile_n(GemmVariant v, bool gateup);
int gemm_w4_tile_n(bool gateup);  // output columns of a W4A16 weight-streaming tile

// K-slices of the router GEMM (partials are summed in slice order by the
// top-k kernel); `partial` needs splits*T*E floats when splits > 1.
int router_splits(int64_t T, int H, int E);
hipError_t launch_router(const uint16_t* x, const float* w, const float* bias, float* logits,
                         float* partial, int32_t* ids, float* wts, int64_t T, int H, int E, int k,
                         float rsf, hipStream_t stream);

// Routing of a batch small enough for one workgroup (T*k <= 4096 pairs and
// T*E <= 16384 logits, decode): the router GEMM, then one kernel that sums
// the logits' K-slice partials into LDS, ranks every token from them (wave
// top-k), permutes the pairs and writes the grouped GEMM's m-tile prefix
// for tiles of bm rows.  Results equal launch_router + launch_permute bit
// for bit.
bool route_small_fits(int64_t T, int E, int k);
hipError_t launch_route_small(const uint16_t* x, const float* w, const float* bias, float* logits,
                              float* partial, int32_t* ids, float* wts, int64_t T, int H, int E,
                              int k, float rsf, int32_t* offsets, int32_t* sorted_token,
                              int32_t* inv_pos, int bm, int32_t* mstart, hipStream_t stream);

int permute_tiles(int64_t N);
// mstart (optional): also write the grouped GEMM's m-tile prefix over the
// expert counts for tiles of bm rows (as launch_gemm_schedule does).
hipError_t launch_permute(const int32_t* ids, int32_t* counts, int32_t* starts, int32_t* offsets,
                          int32_t* sorted_token, int32_t* inv_pos, int64_t N, int E, int k,
                          int bm, int32_t* mstart, hipStream_t stream);

// x_perm[r] = x[sorted_token[r]] for r < N (rows of H bf16, H a multiple of 8).
hipError_t launch_gather_rows(const uint16_t* x, const int32_t* sorted_token, uint16_t* x_perm,
                              int64_t N, int H, hipStream_t stream);

// Tile-blocked copy of G experts' weights for the 256-row tiles: for each
// group, tile b of 256 weight rows and K stage s of 32 columns, one block of
// 256 rows x 32 values (row-contiguous), blocks in the order (group, b, s).
// gate_up (gateup, W [G, 2N, K]): tile b's rows are gate rows 128 b .. + 127
// then the up rows N + 128 b ..; down (W [G, N, K]): rows 256 b .. + 255.
// Rows past N are zeros.  K a multiple of 32.
int64_t pack_experts_elems(int G, int N, int K, bool gateup);
hipError_t launch_pack_experts(const uint16_t* w, uint16_t* packed, int G, int N, int K,
                               bool gateup, hipStream_t stream);

hipError_t launch_gemm_schedule(const int32_t* group_offsets, int G, int bm0, int bm1,
                                int32_t* start0, int32_t* start1, hipStream_t stream);
// max_wgs > 0 caps the persistent weight-streaming grid (default: one
// workgroup per CU), leaving CUs to work on another stream.
hipError_t launch_grouped_gemm(GemmVariant v, bool gateup, const GemmProblem& a,
                               const GemmProblem* b, float limit, hipStream_t stream,
                               int max_wgs = 0);
int gemm_cu_count();  // compute units of the current device

// Router backward (router_bwd.hip): grad_x, grad_w, grad_b each optional
// (NULL skips it); dL element (t, e) at dl[t * rs + e * cs].
size_t router_backward_workspace_bytes(int64_t T, int H, int E);
hipError_t launch_router_backward(const float* dl, int64_t rs, int64_t cs, const uint16_t* x,
                                  const float* w, uint16_t* gx, float* gw, float* gb, int64_t T,
                                  int H, int E, void* ws, hipStream_t stream);

// W4A16 experts -> bf16 (dequant.hip): G groups of `rows` rows by K
// columns (K a multiple of 128), codes [G, rows, K/2], E4M3 scales
// [G, K/128, rows], tensor scales [G] fp32 or nullptr (= 1).
hipError_t launch_w4_dequant(const uint8_t* q, const uint8_t* scale, const float* tscale,
                             uint16_t* out, int G, int64_t rows, int K, hipStream_t stream);

hipError_t launch_rmsnorm_bf16(const uint16_t* x, const float* gamma, uint16_t* out, int64_t T,
                               int H, float eps, hipStream_t stream);
hipError_t launch_combine(const float* y_perm, const float* w, const int32_t* inv_pos,
                          const float* y_shared, const float* gamma_post, const uint16_t* residual,
                          float c0, float c1, uint16_t* out, int64_t T, int H, int k,
                          int post_norm, float eps, hipStream_t stream);

// Device address and size of the current device's copy of the fixed scratch
// (looked up once per device, then cached; noalloc.hip).
hipError_t noalloc_scratch(void** ptr, size_t* bytes);

// Peak probes (probe.hip): a bf16 MFMA throughput kernel (wgs workgroups of
// four wavefronts; sink [wgs * 256] fp32) with its flop count, and an HBM
// read stream over `bytes` (a multiple of 16) of src (sink [wgs * 256]).
hipError_t launch_probe_mfma(int wgs, int iters, float* sink, hipStream_t stream);
double probe_mfma_flops(int wgs, int iters);
hipError_t launch_probe_read(const void* src, int64_t bytes, int wgs, uint32_t* sink,
                             hipStream_t stream);
