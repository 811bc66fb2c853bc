/*
 * woq.h -- C ABI of the MI355X (gfx950) weight-quantisation pass.
 *
 * The pass scores the weight matrices of a model by the Shannon entropy of
 * their softmax (EWQ), tiers the blocks, balances the matrices chosen for
 * low-bit storage with SINQ's alternating row / column standard-deviation
 * scaling, and stores them as group-wise round-to-nearest integer codes packed
 * into bytes (or as ternary {-1, 0, +1} codes with a per-row scale, or as the
 * nearest levels of a non-uniform code book).  The blocks kept in bf16 can be
 * stored with a lossless exponent code.
 *
 * Sources, cited by page title and section:
 *  [EWQ]    "Giai ma EWQ & FastEWQ: Luong tu hoa LLM 'thong minh' hon, nhe hon
 *           ..." (2kvn.com), section "EWQ hoat dong nhu the nao?", steps 1-3.
 *  [SINQ]   "Huawei gioi thieu SINQ: phuong phap luong tu hoa ma nguon mo ..."
 *           (asiadaily.org), sections "Dinh ty le tren hai truc" (dual-axis
 *           scaling), "Chuan hoa Sinkhorn Knopp" and "Tiet kiem bo nho, toc
 *           do va chat luong trong thu nghiem" (non-uniform grids).
 *  [BitNet] "Khung Nguon BitNet.cpp Cua Microsoft ..." (unite.ai), sections
 *           "He Thong Trong So Ternary" and "Luong Tu Hoa Nhom va Chuan Hoa".
 *  [DF11]   "DFloat11: Nen suy luan GPU khong mat du lieu, giam LLM xuong con
 *           70% kich thuoc" (vi.news.hada.io), sections "Dinh dang DFloat11",
 *           "Giai ma dua tren LUT phan cap" and "Kernel GPU hai giai doan va
 *           metadata bo tro" (lossless code for the blocks kept in bf16).
 *
 * Conventions shared by every entry point
 *  - Matrices are row-major, [rows, cols] = [out_features, in_features], with
 *    a row stride `ld` (elements between the starts of consecutive rows):
 *    contiguous (ld = 0 or ld = cols), or ld > cols with ld % 8 == 0 and
 *    cols % 8 == 0 (16-byte rows; for example the q, k or v columns of a fused
 *    [d, 3d] projection weight, or one expert of a [rows, E * cols] tensor);
 *    dtype WOQ_F32 or WOQ_BF16; data 16-byte aligned.  Outputs the library
 *    writes (codes, scales, zero-points) are always contiguous; the lossless
 *    exponent code (df11_*) takes contiguous matrices only.
 *  - Every tensor pointer (inputs, outputs, workspace) is a DEVICE pointer
 *    owned by the caller.  Arrays of descriptors / pointers (the woq_mat
 *    arrays, the `float* const*` style arrays, block_id) are HOST memory read
 *    during the call only.  The library allocates no device memory, keeps no
 *    pointer after the enqueued work completes and has no mutable global
 *    state (except the static scratch array of ewq_block_entropy_static);
 *    calls are thread-safe when they use distinct workspaces.
 *  - Work is enqueued on `stream` (0 = null stream) and the call returns;
 *    outputs are valid once the stream has synchronised.  Calls that share a
 *    workspace must be ordered on one stream.  Every GPU call can be
 *    captured into a HIP graph (stream capture): while the stream is
 *    capturing, the descriptor tables reach the workspace through kernel
 *    arguments instead of a host copy, and only kernels are enqueued (no
 *    memset nodes); a replay repeats the captured call on the same buffers.
 *  - `ws`/`ws_bytes` is a caller-provided device workspace of at least
 *    woq_workspace_size() bytes (256-byte aligned).  Its first WOQ_WS_HEAD
 *    bytes are a status head: ewq_block_entropy and sinq_balance[_ex] write
 *    there, as a uint64 at byte 0, the number of non-finite weights (NaN,
 *    +-inf) among those the call reads (every weight once, however many
 *    iterations), valid once the stream has synchronised.  Other calls leave
 *    the head untouched.
 *  - Every argument error is detected on the host BEFORE anything is
 *    enqueued and before any HIP call; the return value is a WOQ_* status.
 *  - Non-finite weights give NaN entropies / scales and unspecified codes
 *    (and are counted in the workspace head, above).
 *  - Limits: rows, cols >= 1; rows * max(ld, cols) < 2^31 per matrix;
 *    n_mats <= 2^20.  WOQ_ERR_SHAPE otherwise, and for an ld that is neither
 *    0, cols, nor a multiple of 8 above cols (with cols % 8 == 0).
 */
#ifndef WOQ_H_
#define WOQ_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define WOQ_OK            0
#define WOQ_ERR_NULL      1  /* a required pointer is NULL                   */
#define WOQ_ERR_SHAPE     2  /* rows/cols/group/size constraint violated     */
#define WOQ_ERR_DTYPE     3  /* dtype not WOQ_F32 / WOQ_BF16                 */
#define WOQ_ERR_BITS      4  /* bits not in {2, 3, 4, 8} ({2, 3, 4}: code book) */
#define WOQ_ERR_ITERS     5  /* iters < 0 or > 4096                          */
#define WOQ_ERR_WORKSPACE 6  /* ws NULL, misaligned or smaller than needed   */
#define WOQ_ERR_BLOCK     7  /* block id out of range or empty block         */
#define WOQ_ERR_HIP       8  /* a HIP call or kernel launch failed           */
#define WOQ_ERR_ALIGN     9  /* data pointer not 16-byte aligned             */
#define WOQ_ERR_COUNT    10  /* n_mats / n_blocks out of range               */
#define WOQ_ERR_VALUE    11  /* a host-side value is not finite              */
#define WOQ_ERR_SCRATCH  12  /* more than the static scratch array holds     */

/* element types */
#define WOQ_F32  0
#define WOQ_BF16 1

/* bytes at the start of every workspace reserved for the status head */
#define WOQ_WS_HEAD 256

/* operation ids for woq_workspace_size */
#define WOQ_OP_ENTROPY 1
#define WOQ_OP_SINQ    2
#define WOQ_OP_QUANT   3
#define WOQ_OP_DEQUANT 4
#define WOQ_OP_TERNARY 5
#define WOQ_OP_DF11_HIST   6
#define WOQ_OP_DF11_ENCODE 7
#define WOQ_OP_DF11_DECODE 8

/* One matrix.  For dequant_unpack / dequant_codebook / df11_decode it
 * describes the OUTPUT (written). */
typedef struct woq_mat {
    void*   data;      /* device pointer, row-major, 16-B aligned */
    int32_t dtype;     /* WOQ_F32 or WOQ_BF16 */
    int32_t reserved;  /* must be 0 */
    int64_t rows;
    int64_t cols;
    int64_t ld;        /* row stride in elements: 0 or cols (contiguous), or
                          > cols, a multiple of 8 (then cols % 8 == 0) */
} woq_mat;

/* Human-readable name of a status code (static string, never NULL). */
const char* woq_status_string(int32_t status);

/* Workspace bytes needed by operation `op` on these matrices.  `group` is
 * used by WOQ_OP_QUANT / WOQ_OP_DEQUANT only.  WOQ_OP_SINQ covers every
 * sinq_balance_ex flag.  Writes *bytes; returns status. */
int32_t woq_workspace_size(int32_t op, const woq_mat* mats, int32_t n_mats,
                           int32_t group, size_t* bytes);

/*
 * ewq_block_entropy -- [EWQ] steps 1 and 2.
 *  For each matrix m: H_m = -sum p ln p with p = softmax(flatten(W_m)), in
 *  nats (one distribution over all rows*cols entries, the weights are the
 *  logits).  For each block b: H_b = sum n_m H_m / sum n_m over the matrices
 *  with block_id == b (n_m = rows*cols).  Then mu = mean_b H_b, sigma =
 *  population std, T = mu - x*sigma, tier_b = 1 if H_b <= T, else 2 if
 *  H_b < mu, else 3 (with sigma = 0 the first rule wins), and order = block
 *  indices sorted by (H_b, b) ascending.
 *  mats      [n_mats] host array of input matrices (F32 or BF16).
 *  block_id  [n_mats] host array, values in [0, n_blocks); every block must
 *            hold at least one matrix.  NULL means every matrix in block 0
 *            (n_blocks must then be 1).
 *  h_mat     device double[n_mats]            (required)
 *  h_block   device double[n_blocks]          (may be NULL)
 *  stats     device double[3] = {mu, sigma, T} (may be NULL)
 *  tier      device int32[n_blocks]           (may be NULL)
 *  order     device int32[n_blocks]           (may be NULL)
 *  1 <= n_blocks <= 4096.  Results are deterministic (bf16 inputs are
 *  counted exactly by bit pattern; all sums are fp64 in a fixed order).
 *  Speed: a BF16 matrix with many values that are neither zero, NaN / inf
 *  nor of magnitude in [2^-25, 64) (more than 8,192, or more than 240 in
 *  the part one workgroup reads) is recounted with sixteen further reads of
 *  its weights; the results are the same.
 */
int32_t ewq_block_entropy(const woq_mat* mats, int32_t n_mats,
                          const int32_t* block_id, int32_t n_blocks, double x,
                          double* h_mat, double* h_block, double* stats,
                          int32_t* tier, int32_t* order,
                          void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * ewq_block_entropy_ex -- ewq_block_entropy that also writes each BF16
 *  matrix's exponent histogram, taken from the entropy pass's counts with
 *  no further read of the weights: the counts the lossless exponent code of the
 *  blocks the tiers keep is built from ([DF11], "Du dia nen con lai trong
 *  exponent cua BFloat16": the exponent carries far fewer than 8 bits of
 *  information), so df11_build_code needs no df11_exponent_histogram pass.
 *  exp_hist  device uint32[n_mats * 256] (16-B aligned, may be NULL):
 *            exp_hist[i * 256 + e] = number of weights of matrix i whose
 *            exponent field is e (as df11_exponent_histogram); zeros for F32
 *            matrices.
 *  Other arguments, results and errors as for ewq_block_entropy.
 */
int32_t ewq_block_entropy_ex(const woq_mat* mats, int32_t n_mats,
                             const int32_t* block_id, int32_t n_blocks, double x,
                             double* h_mat, double* h_block, double* stats,
                             int32_t* tier, int32_t* order, uint32_t* exp_hist,
                             void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * ewq_block_entropy_static -- ewq_block_entropy for callers that cannot
 *  allocate device memory (code under HIP graph capture, tight serving
 *  loops, harnesses that forbid hipMalloc): no workspace argument, and no
 *  hipMalloc, hipFree or allocating library routine.  Its scratch is a
 *  32 MiB array in the library's device memory, one per GPU the library
 *  runs on (on the device current at the call; `stream` must belong to it),
 *  held until the process ends and located on the first call on each device.
 *  BF16 matrices pass through it in batches of as many as fit (about 48 KB
 *  of counts each), so any number of matrices works; WOQ_ERR_SCRATCH
 *  (before any HIP call) when the descriptor tables, fp32 partials (24
 *  bytes per fp32 work unit: at most 128 units in a matrix of up to 2^26
 *  elements) and the counts of one matrix do not fit (about 400,000 bf16
 *  matrices).  Arguments, results and other errors as for
 *  ewq_block_entropy; the non-finite count is not reported.  Every call on
 *  a GPU uses that GPU's one array: calls that overlap on one GPU (two host
 *  threads, or two streams without ordering between them) race; calls
 *  ordered on one stream do not.
 */
int32_t ewq_block_entropy_static(const woq_mat* mats, int32_t n_mats,
                                 const int32_t* block_id, int32_t n_blocks, double x,
                                 double* h_mat, double* h_block, double* stats,
                                 int32_t* tier, int32_t* order, hipStream_t stream);

/*
 * sinq_balance -- [SINQ] dual-axis scaling by Sinkhorn-Knopp-style
 *  alternating normalisation of row and column standard deviations.
 *  Starting from t = 1, `iters` times:  s_i <- std_j(W_ij / t_j), then
 *  t_j <- std_i(W_ij / s_i); std is the centred population std and a zero
 *  std is replaced by 1.  iters = 0 writes s = t = 1.  The balanced matrix
 *  is W / (s t^T).
 *  row_scale [n_mats] host array of device float[rows]   (s, written)
 *  col_scale [n_mats] host array of device float[cols]   (t, written)
 *  Requires cols % 8 == 0 and cols <= 32768 (WOQ_ERR_SHAPE otherwise: a
 *  row is held by one workgroup).  fp32 element arithmetic with fp64
 *  reductions in a fixed order (deterministic).  The non-finite weights are
 *  counted during the first iteration (workspace head).
 */
int32_t sinq_balance(const woq_mat* mats, int32_t n_mats, int32_t iters,
                     float* const* row_scale, float* const* col_scale,
                     void* ws, size_t ws_bytes, hipStream_t stream);

/* sinq_balance with options.  flags: 0 (as sinq_balance) or a combination of
 *  WOQ_SINQ_RMS     the uncentred root mean square sqrt(mean x^2) in place of
 *                   the centred std in both steps (a zero line gets scale 1),
 *                   for comparing the two readings of the std in a quality
 *                   report;
 *  WOQ_SINQ_SHARED  the call will run concurrently with other work on the
 *                   same GPU (typically a second sinq_balance on another
 *                   stream): row strips are planned for half of the GPU's
 *                   resident workgroups instead of all of them.  Scheduling
 *                   only: the scales are those of the same iteration, with
 *                   column partials summed over different strips (within
 *                   fp32 rounding of the unflagged call; deterministic for a
 *                   given flag).  Each concurrent call needs its own
 *                   workspace.
 *  Other bits: WOQ_ERR_VALUE. */
#define WOQ_SINQ_RMS 1
#define WOQ_SINQ_SHARED 2
int32_t sinq_balance_ex(const woq_mat* mats, int32_t n_mats, int32_t iters, int32_t flags,
                        float* const* row_scale, float* const* col_scale,
                        void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * quant_pack_groupwise -- asymmetric round-to-nearest of the balanced matrix
 *  in groups of `group` consecutive columns of a row (groups are independent,
 *  [BitNet] "Luong Tu Hoa Nhom"), b-bit codes packed LSB-first per row.
 *  With x = (w * (1/s_i)) * (1/t_j) in fp32 (reciprocals correctly rounded;
 *  a NULL array or NULL entry means that scale is 1 and the product is
 *  skipped): lo = min(0, min x), hi = max(0, max x), delta = (hi - lo) /
 *  (2^b - 1), inv = 1/delta, z = clamp(rne(-lo * inv), 0, 2^b - 1),
 *  q = clamp(rne(x * inv) + z, 0, 2^b - 1); every operation is one correctly
 *  rounded fp32 step, round half to even.  A group whose inv is not finite
 *  (delta = 0) gets z = 0 and q = 0.
 *  codes  [n_mats] device uint8[rows * cols * bits / 8]; code of column j in
 *         bits [b*j, b*j + b) of its row's little-endian byte string.
 *  scales [n_mats] device float[rows * cols / group]   (delta, row-major)
 *  zeros  [n_mats] device uint8[rows * cols / group]   (z)
 *  bits in {2, 3, 4, 8}; group % 8 == 0, cols % group == 0; group == 0
 *  means group = cols, one scale per row (EWQ's 8-bit tier).  Groups that
 *  are not a power of two of at most 512 columns are held by one workgroup:
 *  at most 32768 columns for BF16 and 16384 for F32 (WOQ_ERR_SHAPE above,
 *  including group == 0 on wider rows).
 */
int32_t quant_pack_groupwise(const woq_mat* mats, int32_t n_mats,
                             const float* const* row_scale,
                             const float* const* col_scale,
                             int32_t bits, int32_t group,
                             uint8_t* const* codes, float* const* scales,
                             uint8_t* const* zeros,
                             void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * dequant_unpack -- inverse map of quant_pack_groupwise / ternary_pack: the
 *  integer codes back to weights, the reverse of the float -> low-bit
 *  integer mapping of [QG] "Giai thich ve Quantization: huong dan ngan gon
 *  cho LLMs" (kungfutech.edu.vn), section "Luong Tu Hoa La Gi?", with the
 *  balancing undone ([SINQ] "Dinh ty le tren hai truc": W = s t^T o
 *  balanced matrix):
 *  W'_ij = (((q - z) * delta) * s_i) * t_j in fp32 (one rounding per
 *  product), written as F32 or BF16 (round to nearest even) into out[m].
 *  zeros NULL (array or entry) means z = 2^(b-1) - 1 for every group, which
 *  with bits = 2, group = cols and scales = beta decodes ternary codes
 *  ((code - 1) * beta).  row_scale / col_scale as in quant_pack_groupwise.
 */
int32_t dequant_unpack(const woq_mat* out, int32_t n_mats,
                       const uint8_t* const* codes, const float* const* scales,
                       const uint8_t* const* zeros,
                       const float* const* row_scale,
                       const float* const* col_scale,
                       int32_t bits, int32_t group,
                       void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * ternary_pack -- [BitNet] ternary weights {-1, 0, +1} with a per-row scale,
 *  EWQ's 1.58-bit option for its lowest-entropy blocks ([EWQ] step 2).
 *  beta_i = mean_j |W_ij| (fp64 sum, rounded once to fp32); with
 *  inv = 1/beta_i (fp32, correctly rounded) q = clamp(rne(w * inv), -1, 1);
 *  a row with beta = 0 gets q = 0.  Stored as the 2-bit code q + 1,
 *  LSB-first per row (cols / 4 bytes per row).
 *  codes     [n_mats] device uint8[rows * cols / 4]
 *  row_scale [n_mats] device float[rows]  (beta, written)
 *  Requires cols % 8 == 0 and a row held by one workgroup: cols <= 32768
 *  for BF16 and <= 16384 for F32 (WOQ_ERR_SHAPE otherwise).
 */
int32_t ternary_pack(const woq_mat* mats, int32_t n_mats,
                     uint8_t* const* codes, float* const* row_scale,
                     void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * ---- Non-uniform (code-book) grid after balancing ----
 * [SINQ], section "Tiet kiem bo nho, toc do va chat luong trong thu
 * nghiem": the dual-axis scaling also serves non-uniform quantisation.  The
 * page defines no grid; this one scales each group by its largest |x| and
 * maps it to the nearest of 2^b levels given by the caller (for example the
 * normal-quantile levels of woq_codebook_normal).
 *
 * quant_pack_codebook -- with x = (w * (1/s_i)) * (1/t_j) as in
 *  quant_pack_groupwise: a = max |x| over the group, inv = 1/a (0 when not
 *  finite), y = x * inv, code = #{k : y > m_k} with the fp32 midpoints m_k =
 *  (l_k + l_{k+1}) * 0.5 (the nearest level, a tie to the lower one); every
 *  operation one correctly rounded fp32 step.
 *  levels  HOST float[2^bits], finite and strictly ascending (WOQ_ERR_VALUE
 *          otherwise), read during the call.
 *  codes   [n_mats] device uint8[rows * cols * bits / 8], packed as in
 *          quant_pack_groupwise.
 *  scales  [n_mats] device float[rows * cols / group]   (a, row-major)
 *  bits in {2, 3, 4} (WOQ_ERR_BITS otherwise); group rules and workspace
 *  (WOQ_OP_QUANT) as in quant_pack_groupwise.
 */
int32_t quant_pack_codebook(const woq_mat* mats, int32_t n_mats,
                            const float* const* row_scale,
                            const float* const* col_scale,
                            int32_t bits, int32_t group, const float* levels,
                            uint8_t* const* codes, float* const* scales,
                            void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * dequant_codebook -- inverse map of quant_pack_codebook: W'_ij =
 *  ((a * l_q) * s_i) * t_j in fp32 (one rounding per product), written as
 *  F32 or BF16 (round to nearest even) into out[m].  Arguments as in
 *  dequant_unpack (workspace WOQ_OP_DEQUANT) with `levels` as in
 *  quant_pack_codebook and no zero-points.
 */
int32_t dequant_codebook(const woq_mat* out, int32_t n_mats,
                         const uint8_t* const* codes, const float* const* scales,
                         const float* const* row_scale,
                         const float* const* col_scale,
                         int32_t bits, int32_t group, const float* levels,
                         void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * woq_codebook_normal -- the normal-quantile levels for 2^bits codes:
 *  l_k = P((k + 1/2) / 2^bits) / P((2^bits - 1/2) / 2^bits), P the standard
 *  normal quantile (cells of equal probability under N(0, 1), symmetric,
 *  largest level 1), computed in fp64 and rounded to fp32.  Host only:
 *  levels is HOST float[2^bits] (written); bits in {2, 3, 4}.
 */
int32_t woq_codebook_normal(int32_t bits, float* levels);

/*
 * ewq_budget_levels -- [EWQ] step 3 (budgeted placement in the serving
 *  cluster): adjust the precision levels the tiers give so that the model
 *  fits a storage budget.  Host-side only: every pointer is HOST memory and
 *  no GPU work is enqueued.
 *  Levels ascend in storage; level_bytes[b * n_levels + l] is block b's
 *  storage at level l (for example 0 ternary, 1 int4 after balancing,
 *  2 int8 per row, 3 kept bf16).  From level0, with total S:
 *   S <= budget: repeatedly raise by one level the block of highest entropy
 *     (ties: lower index) among those below the top level whose promotion
 *     keeps S <= budget; stop when no promotion fits.
 *   S >  budget: repeatedly lower by one level the block of lowest entropy
 *     (ties: lower index) among those above level 0, until S <= budget or
 *     every block is at level 0.
 *  h_block     [n_blocks] block entropies (finite)
 *  level_bytes [n_blocks * n_levels] (>= 0)
 *  level0      [n_blocks] starting levels in [0, n_levels)
 *  level_out   [n_blocks] (written)   total_out: final bytes (written)
 *  fits_out    1 if the final total is within the budget, else 0 (written)
 *  Errors: NULL pointer (WOQ_ERR_NULL); n_blocks outside [1, 2^20] or
 *  n_levels outside [1, 64] (WOQ_ERR_COUNT); a level0 out of range, a
 *  negative byte count or budget (WOQ_ERR_SHAPE); a non-finite entropy
 *  (WOQ_ERR_VALUE).  Nothing is written on error.
 */
int32_t ewq_budget_levels(const double* h_block, const int64_t* level_bytes,
                          int32_t n_blocks, int32_t n_levels, const int32_t* level0,
                          int64_t budget, int32_t* level_out, int64_t* total_out,
                          int32_t* fits_out);

/*
 * ---- Lossless exponent code for bf16 weights ([DF11]) ----
 *
 * A bf16 word is sign (1 bit), exponent (8) and mantissa (7).  The exponent
 * of each weight is replaced by a prefix code built from the matrix's own
 * exponent histogram; sign and mantissa are kept verbatim.  Format of one
 * encoded matrix of n weights (every byte layout below is exact):
 *  EncodedExponent   the codewords, in weight order, MSB-first (the first
 *                    bit is bit 7 of byte 0); n_seg = ceil(total_bits / 64)
 *                    segments of 8 bytes, buffer 8 n_seg + 8 bytes (zero
 *                    padded).
 *  PackedSignMantissa n bytes, byte i = sign_i << 7 | mantissa_i.
 *  Gaps              per segment t, g_t = (first codeword start >= 64 t, or
 *                    total_bits if none) - 64 t, 0 <= g_t <= 31, packed 5
 *                    bits LSB-first (bits 5t..5t+4 of the array, bit k being
 *                    bit k % 8 of byte k / 8); 4 ceil(5 n_seg / 32) + 4 bytes.
 *  block_pos         n_blocks + 1 uint32, n_blocks = ceil(n_seg / 256):
 *                    block_pos[b] = number of codewords starting before bit
 *                    16384 b (the decoding block of 256 segments), last = n.
 *  tables            n_tables (1..17) x 256 bytes: table 0 is indexed by the
 *                    next 8 stream bits; an entry < 240 is the decoded
 *                    exponent, an entry v >= 240 continues in table 256 - v
 *                    with the following 8 bits.
 *  CodeLengths       256 bytes, the codeword length of each exponent.
 * Code: Huffman code lengths (merge the two nodes of least (count, order);
 * leaves ordered by exponent, internal nodes after every leaf in creation
 * order; a single used exponent gets length 1); when that exceeds 32 bits,
 * the optimal code with lengths <= 32 (package-merge); canonical codewords
 * by (length, exponent).  Exponents >= 240 (|w| >= 2^113, inf, NaN) cannot
 * be coded (those table values are pointers).
 */

/* Sizes of the encoded buffers of a matrix of n weights whose codewords
 * total total_bits (n <= total_bits <= 32 n).  Host-side.  WOQ_ERR_SHAPE on
 * out-of-range arguments. */
int32_t df11_buffer_sizes(int64_t n, int64_t total_bits, int64_t* n_seg,
                          int64_t* enc_bytes, int64_t* gap_bytes, int64_t* n_blocks);

/* Exponent histogram of each matrix: hist[i * 256 + e] = number of weights
 * of matrix i with exponent field e (device uint32[n_mats * 256], 16-B
 * aligned, written).  BF16 only (WOQ_ERR_DTYPE otherwise). */
int32_t df11_exponent_histogram(const woq_mat* mats, int32_t n_mats, uint32_t* hist,
                                void* ws, size_t ws_bytes, hipStream_t stream);

/* The code of one histogram.  Host-side: every pointer is HOST memory.
 *  hist      [256] counts (>= 0)
 *  code_len  [256] written (0 for unused exponents)
 *  codeword  [256] written (right-aligned canonical codewords)
 *  tables    [17 * 256] written; *n_tables of them are used
 *  total_bits = sum hist[e] * code_len[e] (written)
 * WOQ_ERR_VALUE when an exponent >= 240 occurs or the code would need more
 * than 16 sub-tables; WOQ_ERR_SHAPE on negative or oversized counts. */
int32_t df11_build_code(const int64_t* hist, uint8_t* code_len, uint32_t* codeword,
                        uint8_t* tables, int32_t* n_tables, int64_t* total_bits);

/* Encode each matrix with its own code (from df11_build_code on that
 * matrix's histogram).  code_len / codeword: [n_mats] HOST arrays of HOST
 * [256] arrays; total_bits [n_mats] host.  Outputs (device, sized by
 * df11_buffer_sizes, written): enc (16-B aligned), sign_mant (n bytes, 16-B
 * aligned), gaps (16-B aligned), block_pos (4-B aligned).  The codes are
 * checked to be prefix codes without pointer exponents (WOQ_ERR_VALUE); a
 * code or total that does not belong to the data gives unspecified output
 * but every write stays inside the buffers' stated sizes. */
int32_t df11_encode(const woq_mat* mats, int32_t n_mats, const uint8_t* const* code_len,
                    const uint32_t* const* codeword, const int64_t* total_bits,
                    uint8_t* const* enc, uint8_t* const* sign_mant, uint8_t* const* gaps,
                    uint32_t* const* block_pos, void* ws, size_t ws_bytes, hipStream_t stream);

/* Decode a batch of matrices (for example all of one transformer block) back
 * to their exact bf16 words.  out: BF16 matrices (written); enc, sign_mant
 * (16-B aligned), gaps, block_pos (4-B), tables (4-B, n_tables[i] x 256) and
 * code_len (4-B, 256 bytes) are DEVICE arrays per matrix; n_tables and
 * total_bits are HOST arrays.  A corrupt stream gives unspecified weights
 * but no access outside the stated buffers. */
int32_t df11_decode(const woq_mat* out, int32_t n_mats, const uint8_t* const* enc,
                    const uint8_t* const* sign_mant, const uint8_t* const* gaps,
                    const uint32_t* const* block_pos, const uint8_t* const* tables,
                    const int32_t* n_tables, const uint8_t* const* code_len,
                    const int64_t* total_bits, void* ws, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* WOQ_H_ */
