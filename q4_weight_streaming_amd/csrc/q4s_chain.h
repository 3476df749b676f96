// Internal declarations of the chained decode step (q4s_chain.hip), shared
// with the C-ABI host code.
#pragma once

#include "q4s_internal.h"

namespace q4s {

// One matrix of the chained decode step (one token).  Activations that cross
// phases are 64-bit words: fp32 bits in the low half, the step's tag in the
// high half, so a reader can tell this step's value from an older one.
//
// A paired matrix is two matrices of one shape and one activation (gate and
// up) whose row groups alternate in the tile table: virtual row group 2i is
// group i of the first matrix (w), 2i+1 group i of the second (w2).  A tile of
// an even number of groups then holds whole pairs, and its epilogue writes the
// product y * y_b already quantized, as tagged Q8_0 words (yq): the code word
// of rows 4j..4j+3 at yq[j] (the codes' bytes in the low half), the fp32 bits
// of block b's binary16 d_x at yq[rows/4 + b].  The consumer (down) reads them
// through xq.  q hands o its input the same way (yq without w2).
struct ChainMat {
    MatDesc m;            // w and geometry (rows, cols, nb, G, C, ks, dstride), n = 1
    const void* x;        // activation: tagged words [cols], or fp32 when x_plain
    const uint64_t* x2;   // second factor of an elementwise product (tagged), or NULL
    const uint64_t* xq;   // the activation as tagged Q8_0 words of a paired matrix's product, or NULL
    const void* res;      // residual input added to the output: tagged, or fp32 when res_plain; or NULL
    uint64_t* y;          // tagged output [rows], or NULL
    uint64_t* y2;         // tagged res + y [rows] when res
    float* yf;            // plain fp32 output [rows] (the logits), or NULL
    const uint8_t* w2;    // paired: the second matrix's packed weights, else NULL
    uint64_t* y_b;        // paired: tagged output of the second matrix [rows]
    uint64_t* yq;         // tagged Q8_0 words of y * y_b (paired) or of y (q, for o), or NULL
    uint64_t* kpart;      // K-range tiles: tagged fp32 results of K ranges 1..3 [range - 1][G][64], or NULL
    int32_t norm;         // RMS-normalize the activation before quantizing it
    int32_t x_plain, res_plain, pad_;
};

// Parameters of one chained-step launch.
struct ChainParams {
    const ChainMat* mats;
    const uint32_t* tiles;      // (matrix, group set) pairs, phase by phase
    const uint32_t* phase_end;  // cumulative tile count at the end of each phase
    uint32_t* sync;             // error word, then barrier counters (zeroed before every launch)
    uint64_t* trace;            // NULL, or the phase timeline (see q4s_chain_set_trace; 100 MHz clock)
    uint64_t* dump;             // NULL, or the staged Q8_0 inputs [phase][chunk < dump_chunks][lane]
    int32_t dump_chunks;        // chunks per phase in dump (those of the widest activation)
    int32_t n_phases;
    uint32_t gen;               // this step's tag (never 0)
};

// Phase synchronisation of the chained step.
enum ChainSync { kChainCounter = 0, kChainTree = 1, kChainTagged = 2 };
// error line (word 0 error flag, 1 release word, 3 poll limit), top-counter line, 16 sub-counter lines
constexpr int kChainSyncWords = 32 * 18;

// The chained decode step (one cooperative launch; grid = resident workgroups).
hipError_t launch_chain(int sync_mode, const ChainParams& p, int workgroups, uint32_t spin_limit, bool cooperative,
                        hipStream_t st);
constexpr uint32_t kChainDefaultSpin = 1u << 20;
// Tile word: the tile index in bits 0-28; bit 31: one row group whose chunks
// are spread over the 4 waves; bit 30: two row groups, two waves each; bit 29:
// one K range of one row group (index = range * G + group) of a matrix with
// four K splits of at most kChainRangeChunks chunks, its chunks spread over the 4 waves, the
// ranges meeting through kpart (tagged phases only); none: a group set (one
// wave per row group, or per K range).
constexpr uint32_t kChainSplit4 = 1u << 31;
constexpr uint32_t kChainSplit2 = 1u << 30;
constexpr uint32_t kChainRange = 1u << 29;
constexpr uint32_t kChainTileIndex = kChainRange - 1;
constexpr int kChainRangeChunks = 32;  // a K-range tile's chunks at most (its term table)
hipError_t chain_max_workgroups(int sync_mode, int* n);

}  // namespace q4s
