// Internal types shared by the host planner (muon_api.cpp) and the gfx950
// kernels (muon_kernels.hip). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace muon {

// Tile geometry of the two GEMM engines. Workspace matrices are padded to a
// multiple of the tile edge. Padding is zero and stays zero, because every
// epilogue writes 0 outside the valid region.
constexpr int kTileBF16 = 256;  // bf16 engine: 256 x 256 output tiles, K step 64
constexpr int kTileF32 = 128;   // fp32 engine: 128 x 128 output tiles, K step 32
constexpr int kEwTile = 64;     // momentum and apply kernels: 64 x 64 tiles
constexpr int kApplyRows = 16;  // TP shard apply: 16 rows x 1 KB per workgroup
constexpr int kApplyRowBytes = 1024;

// GEMM work queues: one per XCD. Persistent workgroup w serves queue
// w % kQueues first (workgroups are dispatched to the 8 XCDs round-robin), then
// steals from the others. Each queue holds whole blocks of kBlockRows x
// kBlockCols tiles, so concurrently running tiles on one XCD share operand
// panels in that XCD's L2. 4 x 4 tiles: half of an XCD's 32 CUs, the share a
// kernel gets when two chains' kernels run side by side, and also the fastest
// shape for a single chain.
constexpr int kQueues = 8;
constexpr int kBlockRows = 4;
constexpr int kBlockCols = 4;
// bf16 matrices with at most kSmallTileRows tile rows (m <= 4096) take blocks
// of kSmallBlock x kSmallBlock tiles instead: their K loops are shorter (K = m
// for square and update), and a larger block shares each operand slab among
// more tiles. 8 x 8 measured 2.5-3% faster than 4 x 4 on batches of Qwen3-1.7B
// shapes (m = 2048), and with the update engine choice below 1-1.5% faster on
// Qwen3-4B and 8B layer shapes (m = 2560, 4096), while 4 x 4 stays the fastest
// for m = 5120.
constexpr int kSmallTileRows = 16;
constexpr int kSmallBlock = 8;

// One matrix of the batch as the kernels see it. X is the m x n orientation
// of U (m = min(rows, cols)): U itself, or U^T when rows > cols.
struct MatDev {
  void* x[2];         // X ping/pong: mp x np, row-major, leading dimension ldx
  void* a;            // A = X X^T: mp x mp, leading dimension lda
  void* b;            // B = b*A + c*A*A: mp x mp, leading dimension lda
  void* w;            // weights rows x cols (may be null)
  void* delta;        // Delta W rows x cols (may be null)
  const void* g;      // gradient rows x cols
  void* mom;          // momentum rows x cols
  int32_t rows, cols;
  int32_t m, n;       // m = min(rows, cols), n = max(rows, cols)
  int32_t mp, np;     // m, n rounded up to the GEMM tile edge
  int32_t ldx, lda;   // row strides (elements) of X and A/B: the padded width
                      // plus one 128-byte line, so the rows of a tile spread
                      // over all L2 channels
  int32_t tall;       // rows > cols
  int32_t ew_tiles_c; // elementwise tiles along cols: ceil(cols / 64)
  int32_t part_off;   // first norm-partial slot of this matrix
  int32_t n_parts;    // number of elementwise tiles (= partial slots)
  float lr_scale;     // lr * sqrt(max(1, rows / cols))
};

// One output tile of a GEMM phase: matrix index and tile coordinates, and
// for a split-K piece of a Gram tile its K range and partial-sum slot.
struct Tile {
  int32_t mat;
  int32_t ij;    // (ti << 16) | tj
  int32_t kr;    // 0: the whole K range; else (first 256-wide K chunk << 16) | chunks
  int32_t slot;  // split-K piece: its fp32 partial-sum slot (kPartFloats floats); -1: none
};

// A Gram tile split along K runs as pieces, each of which stores its fp32
// partial sums (one 256 x 256 tile, in the accumulator order of the
// four-wave engine) in a slot of the plan's split-K buffer; a reduce launch
// after the Gram launch adds a tile's pieces in piece order and writes A.
constexpr int kPartFloats = 256 * 256;
constexpr int kMaxSplit = 16;  // pieces per tile at most

struct StepCoeffs {
  float a, b, c;  // Newton-Schulz polynomial
  float beta;     // momentum
  float eps;      // norm guard
  int32_t nesterov;
};

// Kernel phases. kUpdateLast is the last iteration's update, which applies the
// step to W (and delta) instead of storing X; it uses the update tile tables.
enum Phase { kGram = 0, kSquare = 1, kUpdate = 2, kUpdateLast = 3 };

// Arguments of one persistent GEMM-phase launch.
struct PhaseArgs {
  const MatDev* mats;
  const Tile* tiles;     // the kQueues per-XCD tile lists of this phase, concatenated
  const int32_t* qoff;   // kQueues + 1 offsets of those lists in `tiles`
  int32_t* counter;      // kQueues queue heads of this launch (zeroed by the momentum kernel)
  const float* scale;  // per-matrix 1/(||U||_F + eps)
  int32_t src;         // ping/pong index read this iteration
  int32_t first;       // first iteration: fold the norm scale in
  int32_t last;        // last iteration: apply to W / delta instead of storing X
  int32_t wf32;        // W and delta are fp32 (fp32 master weights), X, A, B bf16
  StepCoeffs co;
  float* kpart;        // split-K partial sums (Gram); null when the launch has no pieces
};

struct EwArgs {
  const MatDev* mats;
  const int32_t* prefix;  // prefix[i] = first elementwise tile of matrix i; prefix[n] = total
  int32_t n_mats;
  float* partials;        // one fp32 sum of squares per elementwise tile
  int32_t* counters;      // zeroed by the momentum kernel
  int32_t n_counters;
  const float* scale;
  StepCoeffs co;
};

// One view of the TP shard apply (P += D over rows x cols, row strides ldp
// and ldd). The kernel runs one tile of kApplyRows rows x kApplyRowBytes
// bytes per workgroup.
struct ShardDev {
  void* p;
  const void* d;
  int64_t ldp, ldd;
  int32_t rows, cols;
  int32_t tiles_c;  // ceil(cols / tile columns), tile columns = kApplyRowBytes / element size
  int32_t vec;      // cols, ldp, ldd multiples of 16 bytes' worth of elements, both pointers 16-byte aligned
};

// Launchers (muon_kernels.hip). dtype: 0 = fp32, 1 = bf16.
hipError_t launch_momentum(int dtype, const EwArgs& args, int32_t n_blocks, hipStream_t s);
hipError_t launch_norm(const MatDev* mats, const float* partials, float* scale, int32_t n_mats,
                       float eps, hipStream_t s);
hipError_t launch_apply(int dtype, const EwArgs& args, int32_t n_blocks, hipStream_t s);
// blocks workgroups of 256 threads; out holds blocks * 256 floats.
hipError_t launch_mfma_probe(float* out, int32_t blocks, int32_t iters, hipStream_t s);
// prefix[i] = first tile of shard i (prefix[n] = n_blocks).
hipError_t launch_shard_apply(int dtype, const ShardDev* shards, const int32_t* prefix, int32_t n,
                              int32_t n_blocks, hipStream_t s);
// bf16 GEMM engine pipelines: 8 waves of 128 x 64 with K step 64 and a ring
// of 2 LDS stages, or K step 32 and 4 stages; 4 waves of 128 x 128 with K
// step 64 and 2 stages, or K step 32 and 4 stages.
enum GemmVariant { kGemmBK64 = 0, kGemmBK32 = 1, kGemm4W = 2, kGemm4WDeep = 3 };

hipError_t launch_phase(int dtype, int variant, Phase ph, const PhaseArgs& args, int32_t grid,
                        hipStream_t s);
// The reduce launch of a chain's split Gram tiles: list[k] = {mat, ij, pieces,
// first slot} for k < n, one workgroup each (bf16 four-wave engines only).
hipError_t launch_gram_reduce(const PhaseArgs& args, const Tile* list, int32_t n, hipStream_t s);

// Workgroups per CU that the persistent GEMM kernels can keep resident.
int gemm_blocks_per_cu(int dtype, int variant);

// The no-allocation step's workspace: a static device array of kScratchBytes
// per GPU (muon_kernels.hip). scratch_address() gives its device address on
// the current device, looked up once per device.
constexpr size_t kScratchBytes = size_t(64) << 20;
hipError_t scratch_address(void** out);
// dst[0 .. bytes) = 0 (bytes a multiple of 16, dst 16-byte aligned).
hipError_t launch_zero(void* dst, size_t bytes, hipStream_t s);
// Copies bytes from host src to device dst by kernel launches that carry the
// data in their arguments (dst 16-byte aligned; the copy is rounded up to 16
// bytes, so up to 15 bytes past dst + bytes are written with zeros).
hipError_t launch_upload(void* dst, const void* src, size_t bytes, hipStream_t s);

}  // namespace muon
