/*
 * woq.h -- C ABI of the MI355X (gfx950) weight-quantisation pass.
 *
 * The pass scores the weight matrices of a model by the Shannon entropy of
 * their softmax (EWQ), tiers the blocks, balances the matrices chosen for
 * low-bit storage with SINQ's alternating row / column standard-deviation
 * scaling, and stores them as group-wise round-to-nearest integer codes packed
 * into bytes (or as ternary {-1, 0, +1} codes with a per-row scale).
 *
 * Sources, cited by page title and section:
 *  [EWQ]    "Giai ma EWQ & FastEWQ: Luong tu hoa LLM 'thong minh' hon, nhe hon
 *           ..." (2kvn.com), section "EWQ hoat dong nhu the nao?", steps 1-3.
 *  [SINQ]   "Huawei gioi thieu SINQ: phuong phap luong tu hoa ma nguon mo ..."
 *           (asiadaily.org), sections "Dinh ty le tren hai truc" (dual-axis
 *           scaling) and "Chuan hoa Sinkhorn Knopp".
 *  [BitNet] "Khung Nguon BitNet.cpp Cua Microsoft ..." (unite.ai), sections
 *           "He Thong Trong So Ternary" and "Luong Tu Hoa Nhom va Chuan Hoa".
 *
 * Conventions shared by every entry point
 *  - Matrices are row-major, contiguous, [rows, cols] = [out_features,
 *    in_features]; dtype WOQ_F32 or WOQ_BF16; data 16-byte aligned.
 *  - Every tensor pointer (inputs, outputs, workspace) is a DEVICE pointer
 *    owned by the caller.  Arrays of descriptors / pointers (the woq_mat
 *    arrays, the `float* const*` style arrays, block_id) are HOST memory read
 *    during the call only.  The library allocates no device memory, keeps no
 *    pointer after the enqueued work completes and has no mutable global
 *    state; calls are thread-safe when they use distinct workspaces.
 *  - Work is enqueued on `stream` (0 = null stream) and the call returns;
 *    outputs are valid once the stream has synchronised.  Calls that share a
 *    workspace must be ordered on one stream.
 *  - `ws`/`ws_bytes` is a caller-provided device workspace of at least
 *    woq_workspace_size() bytes (256-byte aligned).
 *  - Every argument error is detected on the host BEFORE anything is
 *    enqueued and before any HIP call; the return value is a WOQ_* status.
 *  - Non-finite weights give NaN entropies / scales and unspecified codes.
 *  - Limits: rows, cols >= 1; rows*cols < 2^31 per matrix; n_mats <= 2^20.
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
#define WOQ_ERR_BITS      4  /* bits not in {2, 3, 4, 8}                     */
#define WOQ_ERR_ITERS     5  /* iters < 0 or > 4096                          */
#define WOQ_ERR_WORKSPACE 6  /* ws NULL, misaligned or smaller than needed   */
#define WOQ_ERR_BLOCK     7  /* block id out of range or empty block         */
#define WOQ_ERR_HIP       8  /* a HIP call or kernel launch failed           */
#define WOQ_ERR_ALIGN     9  /* data pointer not 16-byte aligned             */
#define WOQ_ERR_COUNT    10  /* n_mats / n_blocks out of range               */
#define WOQ_ERR_VALUE    11  /* a host-side value is not finite              */

/* element types */
#define WOQ_F32  0
#define WOQ_BF16 1

/* operation ids for woq_workspace_size */
#define WOQ_OP_ENTROPY 1
#define WOQ_OP_SINQ    2
#define WOQ_OP_QUANT   3
#define WOQ_OP_DEQUANT 4
#define WOQ_OP_TERNARY 5

/* One matrix.  For dequant_unpack it describes the OUTPUT (written). */
typedef struct woq_mat {
    void*   data;      /* device pointer, row-major contiguous, 16-B aligned */
    int32_t dtype;     /* WOQ_F32 or WOQ_BF16 */
    int32_t reserved;  /* must be 0 */
    int64_t rows;
    int64_t cols;
} woq_mat;

/* Human-readable name of a status code (static string, never NULL). */
const char* woq_status_string(int32_t status);

/* Workspace bytes needed by operation `op` on these matrices.  `group` is
 * used by WOQ_OP_QUANT / WOQ_OP_DEQUANT only.  Writes *bytes; returns status. */
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
 *  counted exactly in a histogram of their 65,536 bit patterns; all sums are
 *  fp64 in a fixed order).
 */
int32_t ewq_block_entropy(const woq_mat* mats, int32_t n_mats,
                          const int32_t* block_id, int32_t n_blocks, double x,
                          double* h_mat, double* h_block, double* stats,
                          int32_t* tier, int32_t* order,
                          void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * sinq_balance -- [SINQ] dual-axis scaling by Sinkhorn-Knopp-style
 *  alternating normalisation of row and column standard deviations.
 *  Starting from t = 1, `iters` times:  s_i <- std_j(W_ij / t_j), then
 *  t_j <- std_i(W_ij / s_i); std is the centred population std and a zero
 *  std is replaced by 1.  iters = 0 writes s = t = 1.  The balanced matrix
 *  is W / (s t^T).
 *  row_scale [n_mats] host array of device float[rows]   (s, written)
 *  col_scale [n_mats] host array of device float[cols]   (t, written)
 *  Requires cols % 8 == 0.  fp32 element arithmetic with fp64 reductions in
 *  a fixed order (deterministic).
 */
int32_t sinq_balance(const woq_mat* mats, int32_t n_mats, int32_t iters,
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
 *  bits in {2, 3, 4, 8}; group % 8 == 0, cols % group == 0, group <= 32768.
 *  group == cols gives one scale per row (EWQ's 8-bit tier).
 */
int32_t quant_pack_groupwise(const woq_mat* mats, int32_t n_mats,
                             const float* const* row_scale,
                             const float* const* col_scale,
                             int32_t bits, int32_t group,
                             uint8_t* const* codes, float* const* scales,
                             uint8_t* const* zeros,
                             void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * dequant_unpack -- inverse map of quant_pack_groupwise / ternary_pack:
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
 *  Requires cols % 8 == 0.
 */
int32_t ternary_pack(const woq_mat* mats, int32_t n_mats,
                     uint8_t* const* codes, float* const* row_scale,
                     void* ws, size_t ws_bytes, hipStream_t stream);

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

#ifdef __cplusplus
}
#endif

#endif /* WOQ_H_ */
