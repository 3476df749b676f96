// Internal declarations shared by the C-ABI host code and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace q4s {

// Packed Q4_0 geometry.  A 64-row group is one wavefront (lane = row); a chunk
// is 8 blocks = 256 columns.  Per (group, chunk): 8192 nibble bytes laid out
// [block][row][16 B] so one wave-wide 16-byte load reads 1 KB contiguous, then
// 1024 scale bytes [row][8 x binary16] so one 16-byte load per lane fetches the
// lane's 8 scales.
constexpr int kGroupRows = 64;
constexpr int kChunkBlocks = 8;
constexpr int kBlockNibBytes = 16;
constexpr int kChunkNibBytes = kChunkBlocks * kGroupRows * kBlockNibBytes;  // 8192
constexpr int kChunkBytes = kChunkNibBytes + kGroupRows * kChunkBlocks * 2;   // 9216
constexpr int kWaves = 4;                 // wavefronts per workgroup
constexpr int kThreads = kWaves * 64;     // workgroup size
constexpr int kMaxN = 24;                 // activation rows per call (Q4_0 weights)
constexpr int kMaxNQ8 = 8;                // activation rows per call (Q8_0 weights)
constexpr int kTokTile = 8;               // activation rows per MFMA token tile

// Packed Q8_0 geometry.  Same 64-row groups and 8-block chunks; a chunk is
// stored as two pieces of 4 blocks.  Per piece: the int8 values
// [block][half][row][16 B] (8192 B; one wave-wide 16-byte load reads 1 KB
// contiguous), then the scales [row][4 x binary16] (512 B; one 8-byte load per
// lane).
constexpr int kQ8PieceBlocks = 4;
constexpr int kQ8PieceQBytes = kQ8PieceBlocks * 2 * kGroupRows * 16;             // 8192
constexpr int kQ8PieceBytes = kQ8PieceQBytes + kGroupRows * kQ8PieceBlocks * 2;  // 8704
constexpr int kQ8ChunkBytes = 2 * kQ8PieceBytes;                                // 17408

// One matrix as the GEMV kernels see it.  A workgroup tile ("group set") is
// kWaves / ks row groups; the ks waves of one group split its chunks into ks
// contiguous ranges [s*C/ks, (s+1)*C/ks) and add their accumulators in split
// order through LDS.
struct MatDesc {
    const uint8_t* w;     // packed Q4_0
    const int8_t* xq;     // Q8_0 q, int8 [n][cols]
    const uint16_t* xd;   // Q8_0 d_x, binary16 [n][dstride]
    float* y;             // fp32 [n][rows]
    const float* x;       // fp32 activation [n][cols] quantized by the GEMV launch itself, or NULL
    int32_t rows, cols;
    int32_t nb, G, C, ks; // blocks per row, row groups, chunks, K splits (1, 2 or 4)
    int32_t dstride;      // d_x row stride: nb rounded up to a multiple of 8
    int32_t n;            // activation rows
};

// One activation of a batched Q8_0 quantization.
struct QuantDesc {
    const float* x;       // fp32 [n][cols]
    int8_t* q;            // [n][cols]
    uint16_t* d;          // [n][dstride]
    int64_t blk0;         // first global block index of this activation
    int32_t n, cols;
    int32_t dstride;      // nb rounded up to a multiple of 8
    int32_t pad_;
};

// K split chosen from the chunk count alone (so every n and every entry point
// uses the same partition of a given shape).
inline int choose_ksplit(int64_t C) { return C <= 8 ? 1 : (C <= 16 ? 2 : 4); }
inline int64_t dstride_of(int64_t cols) { return (cols / 32 + 7) / 8 * 8; }
inline int64_t groups_of(int64_t rows) { return (rows + kGroupRows - 1) / kGroupRows; }
inline int64_t chunks_of(int64_t cols) { return (cols / 32 + kChunkBlocks - 1) / kChunkBlocks; }
inline int64_t gsets_of(int64_t G, int ks) {
    int gpw = kWaves / ks;
    return (G + gpw - 1) / gpw;
}

// Kernel launchers (q4s_kernels.hip).  Each returns the launch status.
hipError_t launch_repack(const uint8_t* w, uint8_t* packed, int64_t rows, int64_t cols,
                         hipStream_t st);
hipError_t launch_quantize(const QuantDesc& d, hipStream_t st);
constexpr int kQuantTileBlocks = 32;   // Q8_0 blocks per workgroup of the batched quantizer
// n: the sweep's activation rows (non-temporal stores up to kTokTile rows)
hipError_t launch_quantize_batch(const QuantDesc* dev_descs, const uint32_t* dev_tiles, int64_t n_tiles, int n,
                                 hipStream_t st);
hipError_t launch_gemv(const MatDesc& m, int n, int64_t n_gsets, hipStream_t st);
// Tiles are (matrix, group set) pairs; with n == 1 a single-split matrix's tiles are its row groups.
// trace: NULL, or the launch's timeline (kSweepTraceWords words per workgroup, see q4s_sweep_set_trace).
constexpr int kSweepTraceWords = 9;
hipError_t launch_sweep(const MatDesc* dev_mats, const uint32_t* dev_tiles, int64_t n_tiles,
                        int n, uint64_t* trace, hipStream_t st);
hipError_t launch_block_sums(const MatDesc& m, int n, int32_t* s, hipStream_t st);
// 1-row sweeps whose matrices all have one K split: one 8-wave workgroup per (matrix, row group) entry.
hipError_t launch_sweep_split(const MatDesc* dev_mats, const uint32_t* dev_tiles, int64_t n_tiles, bool fused,
                             uint64_t* trace, hipStream_t st);
// The 1-row sweep with the activation quantized by the GEMV waves themselves (tiles as launch_sweep's at n == 1).
hipError_t launch_sweep_fused(const MatDesc* dev_mats, const uint32_t* dev_tiles, int64_t n_tiles,
                              uint64_t* trace, hipStream_t st);
// Q8_0 weights (q4s_q8w.hip).
hipError_t launch_repack_q8_0(const uint8_t* w, uint8_t* packed, int64_t rows, int64_t cols,
                              hipStream_t st);
hipError_t launch_gemv_q8_0(const MatDesc& m, int n, int64_t n_gsets, hipStream_t st);
// 1-row GEMV of a single-split Q8_0 matrix (C <= 8) quantizing m.x into m.xq / m.xd in the same launch.
hipError_t launch_gemv_q8_0_fused(const MatDesc& m, hipStream_t st);
hipError_t launch_block_sums_q8_0(const MatDesc& m, int n, int32_t* s, hipStream_t st);
hipError_t launch_requant_q8_0_to_q4_0(const uint8_t* w8, uint8_t* w4, int64_t n_blocks, hipStream_t st);
// Decode attention (q4s_attn.hip): split-KV partials over 64-position splits, then the combine.
constexpr int kAttnHeadDim = 128;
constexpr int kAttnSplit = 64;
inline int64_t attn_splits(int64_t L) { return (L + kAttnSplit - 1) / kAttnSplit; }
// floats per split in the workspace: n_q*128 outputs, n_q maxima, n_q sums, rounded up to 4
__host__ __device__ inline int64_t attn_split_floats(int64_t n_q) { return (n_q * (kAttnHeadDim + 2) + 3) / 4 * 4; }
hipError_t launch_attn_decode(const float* q, const float* kb, const float* v, float* o, float* ws, int n_q,
                              int n_kv, int64_t L, int64_t l_cap, float scale, hipStream_t st);
// The static scratch of q4s_attn_decode_noalloc: its device address on the current device (looked up
// once per device), or an error.
constexpr size_t kAttnScratchBytes = (size_t)8 << 20;
hipError_t attn_scratch(float** out);
// Grid-barrier measurement (q4s_barrier.hip); kind 0..9 (counter, flags, tree, relaxed-poll counter, spread trees, fence-free variants).
size_t grid_barrier_scratch_words(int n_wg);
hipError_t launch_grid_barrier(int kind, int n_wg, int phases, uint32_t* scratch, hipStream_t st);
hipError_t grid_barrier_max_workgroups(int* n);
hipError_t launch_bench_read(const void* buf, size_t bytes, int lif, int n_blocks,
                             uint32_t* sink, hipStream_t st);
// Reads floor(bytes / unit_bytes) whole units (unit_bytes a multiple of 1024) in the GEMV's wave pattern.
hipError_t launch_bench_read_units(const void* buf, size_t bytes, size_t unit_bytes, uint32_t* sink, hipStream_t st);
hipError_t launch_bench_copy(const void* src, void* dst, size_t bytes, hipStream_t st);

}  // namespace q4s
