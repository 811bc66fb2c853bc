// Host-side launchers implemented by the kernel translation units and used
// by the C-ABI entry points.  Each returns the hipError_t of its launches.
#pragma once

#include "woq_internal.h"

namespace woq {

// ---- entropy ([EWQ] step 1 and 2)
// fp32 work units: at most kEntChunk and at least kEntMinChunk elements,
// a matrix split into about kEntSplit units between these bounds, so that a
// small matrix is still shared among several workgroups.
constexpr int64_t kEntChunk = int64_t(1) << 19;
constexpr int64_t kEntMinChunk = 4096;
constexpr int64_t kEntSplit = 128;
constexpr int kHistSlots = 8192;                   // bf16 matrices per batch
// Per bf16 matrix of a batch: a record of kEntRecWords uint32 (window
// counts and a header; zeroed before counting) and a list of up to
// kEntListCap 16-bit patterns of values outside the window.
constexpr int kEntRecWords = 8128;
constexpr int kEntListCap = 8192;

hipError_t fill_u32(uint32_t* p, size_t n, uint32_t v, hipStream_t s);
// Host bytes to device memory through kernel arguments, kStageChunk bytes
// per launch (n a multiple of 4): safe to capture into a graph.
constexpr int kStageChunk = 2048;
hipError_t stage_bytes(void* dst, const void* src, size_t n, hipStream_t s);
hipError_t fill_f32(float* p, size_t n, float v, hipStream_t s);

// Counting pass over the bf16 matrices mats[0, nmat): vbeg[m] is the first
// 16-byte vector of matrix m in one sequence over the batch (vbeg[nmat] -
// vbeg[0] = n_vec); records and lists indexed by the batch position m.
hipError_t ent_hist_bf16(const EntMat* mats, const int64_t* vbeg, int nmat, int64_t n_vec,
                         uint32_t* recs, uint16_t* lists, hipStream_t s);
// Entropy from the records: one workgroup per matrix.
// nonfinite: the call's uint64 counter of NaN / inf weights (added to).
// exp_hist (may be NULL): per matrix slot 256 exponent-field counts (written).
hipError_t ent_hist_final(const EntMat* mats, int nmat, const uint32_t* recs,
                          const uint16_t* lists, double* h_mat,
                          unsigned long long* nonfinite, uint32_t* exp_hist,
                          hipStream_t s);
// fp32: part holds 3 doubles per work unit; exp_hist (may be NULL): the
// matrices' rows of exponent counts are zeroed.
hipError_t ent_f32(const EntMat* mats, const int64_t* ubeg, int nmat,
                   int64_t n_units, double* part, double* h_mat,
                   unsigned long long* nonfinite, uint32_t* exp_hist, hipStream_t s);
// Blocks per entropy call (the entry points reject more); the tier kernel
// keeps every block entropy in LDS.
constexpr int kMaxBlocks = 4096;
hipError_t ent_blocks(const int32_t* bmats, const int32_t* bbeg,
                      const double* nsz, const double* h_mat, int n_blocks,
                      double x, double* h_block, double* stats,
                      int32_t* tier, int32_t* order, hipStream_t s);

// ---- Sinkhorn ([SINQ])
// Launch shape for a matrix width: mode 1 = one wave per row (rows of at
// most 4096 bf16 / 1536 fp32 columns, nv = vectors per lane), mode 0 = one
// workgroup of nt threads per row strip (nv vectors per thread).
// rag: lanes own unequal numbers of 8-column vectors.
struct SinqShape { int nt, nv, mode, rag; };
SinqShape sinq_shape(int cols, int dtype);
// Rows per register tile of the fused pass (depends on dtype and nv).
int sinq_tile_rows(int dtype, int nv);
// Waves per SIMD the wave-per-row pass is built for (dtype, vectors per lane).
int sinq_wave_occupancy(int dtype, int nv);
// Column reduction: slices of partial rows per column (a power of two, 1..16)
// for a launch whose matrices have at most max_strips partial rows; a
// reduction workgroup covers 256 / slices columns.
int sinq_reduce_slices(int max_strips);
// One iteration over a group of same-shape matrices: the fused row / column
// pass then the fixed-order column reduction.  A wave-form matrix swept by
// a single workgroup (n_strips == 1) has its columns finished by that
// workgroup and no units in col_begin; n_col_units == 0 launches no
// reduction.  The first iteration adds the
// NaN / inf weights it reads to *nonfinite.
hipError_t sinq_iteration(const SinqMat* mats, const int64_t* strip_begin,
                          const int64_t* col_begin, int nmat, int64_t n_strips,
                          int64_t n_col_units, int max_strips, int dtype, SinqShape sh,
                          int cols_max, bool first, unsigned long long* nonfinite,
                          hipStream_t s);

// ---- quantise / dequantise / ternary

struct RecipSeg {
    const float* src;
    float* dst;
    int64_t n;
    int64_t unit_begin;               // units of 256 elements
};
hipError_t recip(const RecipSeg* segs, const int64_t* ubeg, int nseg,
                 int64_t n_units, hipStream_t s);
// Group kinds of quant_pack_groupwise: tiles of kQTileRows x kQTileCols for
// power-of-two groups of at most 512 columns, one wave per group up to
// kQWaveMax columns, else one workgroup per group.
constexpr int kQTileRows = 8;
constexpr int kQTileCols = 2048;
constexpr int kQWaveMax = 4096;
// dequant_unpack tiles: kDTileRows x kQTileCols (any group).
constexpr int kDTileRows = 4;
// book == NULL: the affine grid; else the code-book grid (bits 2..4) with
// the table at `book` in device memory and `steps` comparisons per value.
// tie: some matrix of the launch has no scales, or bits == 8, so element
// ratios near a half-way point must be re-decided by division (affine grid).
hipError_t quant_tile(const QMat* mats, const int64_t* ubeg, int nmat,
                      int64_t n_units, int dtype, int bits, const CbTable* book,
                      int steps, bool tie, hipStream_t s);
hipError_t quant_wave(const QMat* mats, const int64_t* ubeg, int nmat,
                      int64_t n_units, int dtype, int bits, int nvl,
                      const CbTable* book, int steps, bool tie, hipStream_t s);
hipError_t quant_big(const QMat* mats, const int64_t* ubeg, int nmat,
                     int64_t n_units, int dtype, int bits, const CbTable* book,
                     int steps, bool tie, hipStream_t s);
hipError_t dequant(const QMat* mats, const int64_t* ubeg, int nmat,
                   int64_t n_units, int out_dtype, int bits, const CbTable* book,
                   hipStream_t s);
// Ternary, rows of at most kTernWaveMax columns: one wave per row,
// kTernRows rows per unit; nvl = 8-column vectors per lane (1, 2, 4 or 8).
constexpr int kTernRows = 16;
constexpr int kTernWaveMax = 4096;
hipError_t ternary_wave(const QMat* mats, const int64_t* ubeg, int nmat, int64_t n_units,
                        int dtype, int nvl, hipStream_t s);
// Ternary, wider rows: one workgroup per row (one unit per row).
hipError_t ternary(const QMat* mats, const int64_t* ubeg, int nmat,
                   int64_t n_units, int dtype, hipStream_t s);

// ---- lossless exponent code (DF11)
// Host: code lengths, canonical codewords and hierarchical tables from an
// exponent histogram (tables: up to (kDf11MaxSub + 1) * 256 bytes).
int32_t df11_code_build(const int64_t* hist, uint8_t* code_len, uint32_t* codeword,
                        uint8_t* tables, int32_t* n_tables, int64_t* total_bits);
// Exponent histograms (hist[nmat * 256], zeroed by the caller); units of
// kDf11Chunk weights.
hipError_t df11_hist(const DfMat* mats, const int64_t* ubeg, int nmat, int64_t n_units,
                     uint32_t* hist, hipStream_t s);
// Encode: ubeg has nmat + 1 entries (units of kDf11Chunk weights); zbeg
// covers the stream and gap words to clear (units of 4096 words).
hipError_t df11_encode_run(const DfMat* mats, const int64_t* ubeg, int nmat, int64_t n_units,
                           const int64_t* zbeg, int64_t n_zunits, const DfCode* codes,
                           uint32_t* chunk_bits, int64_t* chunk_base, hipStream_t s);
// Decode: one unit per decoding block.
hipError_t df11_decode_run(const DfMat* mats, const int64_t* ubeg, int nmat, int64_t n_units,
                           hipStream_t s);

}  // namespace woq
