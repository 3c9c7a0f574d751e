/*
 * w4a16.h -- C ABI of the W4A16 skinny matmul for speculative-verify decode
 * (AMD Instinct MI355X, gfx950).
 *
 * The operation.  Single-stream decode reads every weight once per cycle and
 * verifies T = 1 + n_draft tokens against it (qwen-warp/llamAmpere article,
 * "The arithmetic every claim answers to": a decode step lasts as long as
 * reading the weights takes, so scoring several drafted tokens costs about
 * as much as one token when each weight is read a single time for the whole
 * block of T rows).  Weights are W4A16 with group 128, in the
 * format that article describes under "qwen-warp: keep the activations in
 * bf16": 4-bit codes packed as little-endian words of eight nibbles, level =
 * code - 8, one bf16 scale per 128 columns of a row.  For T activation rows
 * x (bf16) the library computes, in fp32,
 *
 *     y[t][n] = sum_k (q[n][k] - 8) * scale[n][k/128] * x[t][k].
 *
 * Each level (q - 8) and each product with x is formed exactly, for every
 * finite bf16 x: the matrix cores multiply exact levels with the staged
 * activations, as fp16 times a power of two where every value of the staged
 * block converts exactly, else as the bf16 values they are; sums are fp32
 * (scaled by that power of two and back, which rounds as the unscaled sums
 * would), with a fresh partial per 128-column group
 * multiplied by that group's scale (the same section: the scale multiplies,
 * in fp32, the sum of the group's products).  Results agree with the exact
 * sum within 1e-3 * sum_k |w*x| + 1e-6 per element, for any finite inputs
 * whose partial sums stay inside the fp32 range (beyond about 3.4e38 a sum
 * overflows to infinity, as the fp32 output itself must).
 *
 * Layout (all row-major, all device memory owned by the caller):
 *   packed_u4    uint8   [rows][K/2]    byte j of a row holds column 2j in bits
 *                                       0-3 and column 2j+1 in bits 4-7
 *   scales_bf16  uint16  [rows][K/128]  bf16 bit patterns
 *   x_bf16       uint16  [T][K]         bf16 bit patterns
 *   y_f32        float   [T][n_out]
 *
 * Conventions for every entry point:
 *   - All work is enqueued on `stream` (0 = the null stream); the call returns
 *     before the GPU finishes.  Results are valid after the caller synchronises.
 *   - All arguments are checked on the host before anything is enqueued; on
 *     any status other than W4A16_OK and W4A16_ERR_HIP nothing was enqueued.
 *     W4A16_ERR_HIP means a HIP runtime call failed (the launch itself or a
 *     device query).
 *   - No allocation, no synchronisation, no printing, and no state kept
 *     between calls apart from the process-wide variant selection
 *     (w4a16_set_variant), the measurement tile override (w4a16_set_tile)
 *     and the static argmax scratch of w4a16_head_gather_noalloc.  Outputs
 *     must not alias inputs or each other.
 *   - Thread-safe; calls on different streams may run concurrently.
 *   - Activations should be finite; a non-finite x gives non-finite outputs
 *     for the rows it reaches.
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#ifndef HIP_INCLUDE_HIP_HIP_RUNTIME_API_H
typedef struct ihipStream_t* hipStream_t; /* same definition as the HIP runtime's */
#endif

#define W4A16_GROUP 128      /* columns per bf16 scale */
#define W4A16_MAX_T 16       /* activation rows per weight read */
#define W4A16_ABI_VERSION 6

typedef enum {
  W4A16_OK = 0,
  W4A16_ERR_NULL_POINTER = 1, /* a required pointer is NULL */
  W4A16_ERR_BAD_SHAPE = 2,    /* a size is out of range (see each call) */
  W4A16_ERR_MISALIGNED = 3,   /* packed_u4 / x_bf16 not 16-byte aligned, scales not 2, y / ids / argmax not 4 */
  W4A16_ERR_WORKSPACE = 4,    /* argmax workspace (or batch table buffer) missing or too small */
  W4A16_ERR_UNSUPPORTED = 5,  /* the current device is not gfx950 */
  W4A16_ERR_HIP = 6,          /* a HIP runtime call returned an error */
  W4A16_ERR_BAD_VARIANT = 7,  /* unknown kernel variant */
  W4A16_ERR_SCRATCH = 8       /* w4a16_head_gather_noalloc: argmax partials larger than its static scratch */
} w4a16_status;

/* Kernel variants.  Both compute the same values within the tolerance above.
 * AUTO runs the matrix-core kernels: on MI355X they are faster on every
 * workload shape at every T.  The dot variant covers T <= 8; calls with more
 * activation rows run the matrix-core kernels whatever the selection. */
typedef enum {
  W4A16_VARIANT_AUTO = 0,
  W4A16_VARIANT_DOT = 1, /* VALU bf16 dot products, split-K across lanes, cross-lane reduction */
  W4A16_VARIANT_MFMA = 2 /* bf16 matrix cores, tokens padded to 16 rows */
} w4a16_variant;

/*
 * y = x * W^T for one weight matrix.
 *   N  output rows, 1 <= N <= 2^31-1
 *   K  reduction length, a multiple of 128, 128 <= K <= 2^20
 *   T  activation rows, 1 <= T <= W4A16_MAX_T
 */
w4a16_status w4a16_matmul(const uint8_t* packed_u4, const uint16_t* scales_bf16, const uint16_t* x_bf16,
                          float* y_f32, int64_t N, int64_t K, int32_t T, hipStream_t stream);

/*
 * Scores a subset of the rows of an output head (e.g. the lm_head) and
 * optionally takes the per-row argmax.  Follows the draft head of the
 * swift-qwen3.8-rtx3090 project page ("Body, heads and drafter": the
 * drafter's head keeps only the lm_head rows of the draft vocabulary) and the
 * OpenJet engine page ("How it gets its speed": the drafter scores a token
 * list, verification every vocabulary id).
 *
 *   row_ids   int32 [n_ids] device ids into [0, n_rows); output row i uses
 *             weight row row_ids[i].  NULL means the identity, n_ids = n_rows
 *             (the full head).  Duplicates are allowed.  An id outside
 *             [0, n_rows) yields a NaN output row that never wins the argmax.
 *   y_f32     [T][n_ids] in row_ids order, or NULL to skip writing scores.
 *   argmax_id [T] or NULL (no argmax); argmax_val [T] or NULL (needs
 *             argmax_id).  For each t: the largest
 *             non-NaN score and the lowest vocabulary id (row_ids value)
 *             attaining it; greedy verification accepts a draft when it
 *             equals this argmax (qwen-warp/llamAmpere article, "What each
 *             one calls the same answer").  No valid row: id -1, value NaN.
 *   workspace device scratch of at least w4a16_workspace_bytes(n_ids, T) bytes
 *             (16-byte aligned), required when argmax is requested; its
 *             contents need no initialisation and are meaningless afterwards.
 *   Shapes: 1 <= n_ids, n_rows <= 2^31-1; K and T as for w4a16_matmul.
 *   At least one of y_f32 and argmax_id must be non-NULL.
 */
w4a16_status w4a16_head_gather(const int32_t* row_ids, int64_t n_ids, const uint8_t* packed_u4,
                               const uint16_t* scales_bf16, int64_t n_rows, const uint16_t* x_bf16, int64_t K,
                               int32_t T, float* y_f32, int32_t* argmax_id, float* argmax_val, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes w4a16_head_gather needs for n_out scored rows at T
 * (0 for arguments out of range). */
size_t w4a16_workspace_bytes(int64_t n_out, int32_t T);

/*
 * w4a16_head_gather without a workspace argument and without any
 * allocation, for callers that cannot allocate device memory: code being
 * captured into a HIP graph, tight serving loops, harnesses that forbid
 * hipMalloc.  The argmax partials go to a static device array of
 * W4A16_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends; its device address is looked up once per device
 * (hipGetSymbolAddress).  Same arguments, kernels and results as
 * w4a16_head_gather otherwise.
 *   Limit: with argmax_id set, w4a16_workspace_bytes(n_ids, T) must not
 *   exceed W4A16_NOALLOC_SCRATCH_BYTES (2 MiB: e.g. 262,144 rows at T = 16,
 *   enough for a 248,320-row vocabulary head), else W4A16_ERR_SCRATCH and
 *   nothing is enqueued.  Without argmax the array is not used.
 *   The array needs no initialisation (each workgroup writes its own
 *   partials before the reduction reads them) and keeps the last call's
 *   contents.  Every call on one GPU shares it: calls that may overlap on
 *   one GPU (different streams, or different host threads) race and must be
 *   serialised by the caller.
 */
#define W4A16_NOALLOC_SCRATCH_BYTES (2u << 20)

w4a16_status w4a16_head_gather_noalloc(const int32_t* row_ids, int64_t n_ids, const uint8_t* packed_u4,
                                       const uint16_t* scales_bf16, int64_t n_rows, const uint16_t* x_bf16,
                                       int64_t K, int32_t T, float* y_f32, int32_t* argmax_id, float* argmax_val,
                                       hipStream_t stream);

/*
 * Tiled weight layout: a one-time repack of the same codes and scales so
 * that each group of 16 rows x 128 columns is one contiguous 1 KB block and
 * each row's scales travel with its codes.  Follows the OpenJet engine page
 * ("How it gets its speed"), whose engine rearranges some weight formats a
 * single time when the model loads -- the numbers stay the same -- so that
 * the loads are wide and aligned and the scales come in the same block as
 * the codes.  On MI355X a wave's 16-byte-per-lane load then covers one
 * contiguous 1 KB block instead of 64 bytes of 16 rows.
 *
 * Definition (G = K/128 groups, rows padded to a multiple of 16 with zero
 * bytes): for tile i (rows 16i .. 16i+15), chunk c (groups 8c .. 8c+ng-1,
 * ng = min(8, G - 8c)), group g of the chunk and row r of the tile:
 *   tile i starts at byte   i * w4a16_tiled_tile_bytes(K)
 *   chunk c starts at byte  c * (8 * 1024 + 256) within the tile
 *   codes of (g, r): 64 bytes at  chunk + (g - 8c) * 1024 + 64 * r, equal to
 *                    bytes 64g .. 64g+63 of row 16i + r in packed_u4
 *   scales of (c, r): 16 bytes at chunk + ng * 1024 + 16 * r: the bf16 scales
 *                    of groups 8c .. 8c+7 of row 16i + r (zero past G)
 * so a tile takes G * 1024 + ceil(G/8) * 256 bytes (0.515625 B per weight
 * when G % 8 == 0, the same as the row-major pair).
 */

/* Bytes per 16-row tile, and of the whole tiled layout (0 if out of range). */
size_t w4a16_tiled_tile_bytes(int64_t K);
size_t w4a16_tiled_bytes(int64_t N, int64_t K);

/*
 * Writes the tiled layout of a row-major weight (packed_u4 [N][K/2],
 * scales_bf16 [N][K/128]) into `tiled` (device, 16-byte aligned, at least
 * w4a16_tiled_bytes(N, K) bytes, must not overlap the inputs).  Shapes as
 * for w4a16_matmul.  W4A16_ERR_WORKSPACE if tiled_bytes is too small.
 */
w4a16_status w4a16_repack_tiled(const uint8_t* packed_u4, const uint16_t* scales_bf16, int64_t N, int64_t K,
                                void* tiled, size_t tiled_bytes, hipStream_t stream);

/*
 * The tiled layout of a subset of a weight's rows: output row i holds input
 * row row_ids[i] of packed_u4 [n_rows][K/2] / scales_bf16 [n_rows][K/128].
 * For a head restricted to a fixed id list (the swift-qwen3.8-rtx3090 page,
 * "Body, heads and drafter": the drafter's head keeps only the lm_head rows
 * of the draft vocabulary), built once at load: the subset is then a plain
 * tiled matrix of n_ids rows, read in whole 1 KB blocks instead of 64-byte
 * pieces of scattered rows.  Scores and argmax of calls on it are by
 * position i; the vocabulary id is row_ids[i] (with row_ids in ascending
 * order, the lowest-position tie rule is the lowest-id rule).
 *   row_ids  int32 [n_ids] device, each in [0, n_rows); duplicates allowed.
 *            An id outside gives a row of zero codes and NaN scales, whose
 *            scores are NaN and never win an argmax (as the same id does in
 *            w4a16_head_gather).
 *   tiled    device, 16-byte aligned, >= w4a16_tiled_bytes(n_ids, K) bytes.
 *   Shapes: 1 <= n_rows, n_ids <= 2^31-1; K as for w4a16_matmul.
 */
w4a16_status w4a16_repack_tiled_rows(const uint8_t* packed_u4, const uint16_t* scales_bf16, int64_t n_rows, int64_t K,
                                     const int32_t* row_ids, int64_t n_ids, void* tiled, size_t tiled_bytes,
                                     hipStream_t stream);

/* w4a16_matmul and w4a16_head_gather on a tiled weight (`tiled` 16-byte
 * aligned, written by w4a16_repack_tiled for the same N / n_rows and K).
 * Same results within the tolerance; always the matrix-core kernels. */
w4a16_status w4a16_matmul_tiled(const void* tiled, const uint16_t* x_bf16, float* y_f32, int64_t N, int64_t K,
                                int32_t T, hipStream_t stream);
w4a16_status w4a16_head_gather_tiled(const int32_t* row_ids, int64_t n_ids, const void* tiled, int64_t n_rows,
                                     const uint16_t* x_bf16, int64_t K, int32_t T, float* y_f32, int32_t* argmax_id,
                                     float* argmax_val, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream);

/*
 * Grouped launch: many independent matmuls with the same T in one kernel
 * launch, so a whole decode weight pass (e.g. 64 layers x 4 projections) runs
 * without launch gaps or per-kernel ramp-up and tail.  The pages run a verify
 * cycle as one CUDA graph (qwen-warp section) or one persistent launch
 * (OpenJet engine page, "How it works"), and name ~1300 small launches per
 * token as the P100 build's decode bottleneck (P100 patch page, "Persistent
 * layer kernels").
 *
 * Use: w4a16_batch_plan() (host only, no HIP call) checks every problem and
 * writes a launch table into caller-owned host memory of
 * w4a16_batch_table_bytes(count) bytes; the caller copies those bytes to
 * device memory (16-byte aligned) and then calls w4a16_matmul_batch() with
 * both copies, as often as it likes.  The device copy must hold exactly the
 * bytes of the host copy and stay unchanged while launches that use it run.
 * Problems run in list order as far as the GPU schedules them; their outputs
 * must not overlap each other or any input.  The pointers and sizes of each
 * problem follow w4a16_matmul.  A problem may also take the per-row argmax
 * of its outputs, as w4a16_head_gather does (the lm_head of a verify pass in
 * the same launch as the layers; the argmax reduction then runs as one small
 * launch per such problem after the grouped one, on the same stream).
 */
typedef struct {
  const uint8_t* packed_u4;    /* [N][K/2], or the tiled layout when layout = 1 */
  const uint16_t* scales_bf16; /* [N][K/128]; ignored (may be NULL) when layout = 1 */
  const uint16_t* x_bf16;      /* [T][K] */
  float* y_f32;                /* [T][N] */
  int64_t N;
  int64_t K;
  int32_t layout;              /* W4A16_LAYOUT_ROW_MAJOR or W4A16_LAYOUT_TILED */
  int32_t reserved;            /* must be 0 */
  int32_t* argmax_id;          /* [T] device, or NULL: no argmax for this problem */
  float* argmax_val;           /* [T] device, or NULL (needs argmax_id) */
  void* workspace;             /* with argmax_id: device, 16-byte aligned, at least */
  size_t workspace_bytes;      /*   w4a16_workspace_bytes(N, T) bytes, one per problem */
} w4a16_problem;

#define W4A16_LAYOUT_ROW_MAJOR 0
#define W4A16_LAYOUT_TILED 1

#define W4A16_MAX_BATCH 65536

/* Table bytes for `count` problems (0 if count is out of [1, W4A16_MAX_BATCH]). */
size_t w4a16_batch_table_bytes(int32_t count);

w4a16_status w4a16_batch_plan(const w4a16_problem* problems, int32_t count, int32_t T, void* table_host,
                              size_t table_bytes);

/* W4A16_ERR_BAD_SHAPE if table_host is not a table written by w4a16_batch_plan. */
w4a16_status w4a16_matmul_batch(const void* table_host, const void* table_dev, hipStream_t stream);

/*
 * The grouped launch with a device workspace for the activations.  No
 * plan needs one: the workgroups stage every problem's activations into LDS
 * themselves, so w4a16_batch_workspace_bytes returns
 * 0 for every table (and for anything that is not a table), the workspace
 * arguments of w4a16_matmul_batch_ws are ignored (NULL and 0 are fine), and
 * the call is w4a16_matmul_batch.  Kept so that callers written against the
 * workspace form keep working.
 */
size_t w4a16_batch_workspace_bytes(const void* table_host);
w4a16_status w4a16_matmul_batch_ws(const void* table_host, const void* table_dev, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream);

/*
 * Verify epilogue: what a speculative cycle does with the head's scores
 * before the host reads anything back (OpenJet engine page, "How it works":
 * verification on the device, only the accepted tokens go to the host).
 *
 * Per-row top-k.  The OpenJet page ("How it gets its speed") hands its
 * sampler the highest 32 scores of every row it verifies; the qwen-warp
 * article ("What each one calls the same answer") rescores the 16 highest
 * candidates of the quantized head.  For each activation row t of scores [T][n] (e.g. the y
 * of w4a16_head_gather): the k largest non-NaN scores and their vocabulary
 * ids, score descending, equal scores by ascending id, so entry 0 is the
 * argmax of w4a16_head_gather.  -0 and +0 are equal.  Position i has
 * vocabulary id row_ids[i] (NULL: i); a NaN score or a negative id never
 * counts.  With fewer than k countable entries the rest of the row is id -1,
 * value NaN.
 *   scores    float [T][n] device; 1 <= n <= 2^31-1, 1 <= T <= W4A16_MAX_T
 *   row_ids   int32 [n] device or NULL
 *   k         1 <= k <= W4A16_MAX_TOPK
 *   top_ids   int32 [T][k] device (required); top_vals float [T][k] or NULL
 *   workspace device, 16-byte aligned, at least
 *             w4a16_topk_workspace_bytes(n, T, k) bytes (no initialisation)
 */
#define W4A16_MAX_TOPK 32

size_t w4a16_topk_workspace_bytes(int64_t n, int32_t T, int32_t k);

w4a16_status w4a16_topk(const float* scores, int64_t n, int32_t T, const int32_t* row_ids, int32_t k,
                        int32_t* top_ids, float* top_vals, void* workspace, size_t workspace_bytes,
                        hipStream_t stream);

/*
 * Greedy acceptance (qwen-warp article, "What each one calls the same
 * answer": under greedy decoding a draft is kept when it equals the target
 * model's argmax on its verify row).
 * n_seq sequences of `rows` verify rows each, e.g. the T = n_seq * rows rows
 * of one head call.  Row r of sequence s carries the target model's greedy
 * choice target_ids[s*rows + r] (the argmax ids of w4a16_head_gather) for
 * the token after position r; draft_ids[s*(rows-1) + j] is the drafted token
 * that was the input of row j+1.  Draft j is accepted when drafts 0..j-1
 * were and target_ids[s*rows + j] equals it (a negative target id never
 * matches).  n_accepted[s] = a, the accepted drafts; tokens[s*rows + r] =
 * target_ids[s*rows + r] for r <= a (the accepted drafts followed by the
 * target model's next token) and -1 after.
 *   target_ids int32 [n_seq*rows] device; draft_ids int32 [n_seq*(rows-1)]
 *   device (may be NULL when rows = 1); n_accepted int32 [n_seq] device;
 *   tokens int32 [n_seq*rows] device or NULL.
 *   1 <= n_seq <= W4A16_MAX_BATCH, 1 <= rows <= W4A16_MAX_T.
 */
w4a16_status w4a16_greedy_accept(const int32_t* target_ids, const int32_t* draft_ids, int32_t n_seq, int32_t rows,
                                 int32_t* n_accepted, int32_t* tokens, hipStream_t stream);

/*
 * Draft-head id list with the sequence's tokens (OpenJet engine page, "How
 * it gets its speed": the drafter's head scores a fixed list of 32,768
 * common tokens, extended at run time by whichever ids of the current
 * sequence the list lacks, while verification scores every vocabulary id).  Writes into
 * union_ids [n_base + n_seq]: base_ids verbatim, then every id of seq_ids in
 * order of first appearance that lies in [0, n_rows) and is neither in the
 * base list nor already added, then -1 in the remaining slots; *n_union (one
 * int32 on the device) receives the length of the list.  Built for one
 * gathered pass of known size: w4a16_head_gather with row_ids = union_ids
 * and n_ids = n_base + n_seq scores the list, the -1 slots giving NaN rows
 * that no argmax or top-k counts (their loads all hit one cached row).
 *   base_ids int32 [n_base] device (NULL when n_base = 0), taken as given;
 *   seq_ids int32 [n_seq] device (NULL when n_seq = 0), any values;
 *   0 <= n_seq <= W4A16_MAX_SEQ_IDS, 0 <= n_base, 1 <= n_base + n_seq <= 2^31-1,
 *   1 <= n_rows <= W4A16_MAX_UNION_VOCAB.
 */
#define W4A16_MAX_SEQ_IDS 4096
#define W4A16_MAX_UNION_VOCAB 524288

w4a16_status w4a16_draft_union(const int32_t* base_ids, int32_t n_base, const int32_t* seq_ids, int32_t n_seq,
                               int64_t n_rows, int32_t* union_ids, int32_t* n_union, hipStream_t stream);

/* Measurement helper (not a step of the path): reads `bytes` of device
 * memory at src once with 16-byte nontemporal loads spread over
 * `workgroups` workgroups of 256 threads, each taking one contiguous share,
 * and writes one XOR-folded word per thread to sink.  Its rate is the
 * achievable streaming-read ceiling that the matmul's weight bandwidth is
 * set beside (the peak it is measured against stays the nominal 8 TB/s).
 *   src 16-byte aligned, bytes a positive multiple of 16;
 *   sink uint32 [workgroups * 256] device, 4-byte aligned;
 *   1 <= workgroups <= 65536.
 */
w4a16_status w4a16_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t workgroups,
                               hipStream_t stream);

/* Measurement helper (not a step of the path): replaces the planner's tile
 * choice for subsequent calls in this process, of single launches (batch 0)
 * or grouped launches (batch 1), by spec = "split,rt,waves" or
 * "shared,rt,waves" (rt 1, 2 or 4; waves 1-8, or 1-16 for shared workgroups
 * of one tile) or "run,tiles,waves" (tiles per wave 1-16, waves 1-16; a
 * grouped launch mixing both layouts takes shared workgroups of one tile
 * per wave with that many waves instead); NULL or "" restores the planner's
 * choice.  The environment variables
 * W4A16_TILE and W4A16_BATCH_TILE, read once per process, set the initial
 * overrides.  Results stay within the tolerance whatever the tiling.
 * W4A16_ERR_BAD_SHAPE for a batch value or spec that does not parse. */
w4a16_status w4a16_set_tile(int32_t batch, const char* spec);

/* Selects the kernel variant for subsequent calls in this process (initially
 * taken from the environment variable W4A16_VARIANT = auto|dot|mfma). */
w4a16_status w4a16_set_variant(int32_t variant);
int32_t w4a16_get_variant(void);

const char* w4a16_status_string(int32_t status);
int32_t w4a16_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
