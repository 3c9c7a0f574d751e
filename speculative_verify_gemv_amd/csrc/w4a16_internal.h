// Internal interface between the C-ABI layer (w4a16_api.hip) and the gfx950
// kernels (w4a16_kernels.hip).  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a16 {

// One weight matrix (or a gathered subset of its rows) against T activation
// rows, with the tiling the planner chose.  Also the entry type of the device
// table of a grouped launch.
struct GemvArgs {
  const uint8_t* packed;   // [n_rows][K/2]
  const uint16_t* scales;  // [n_rows][K/128] bf16 bits
  const uint16_t* x;       // [T][K] bf16 bits
  float* y;                // [T][n_out] or nullptr
  const int32_t* row_ids;  // [n_out] or nullptr (identity)
  int2* partial;           // argmax partials [workgroups][T] (value bits, id) or nullptr
  int64_t n_out;
  int64_t n_rows;
  int64_t wg_start;        // first workgroup of this problem in a grouped launch
  int32_t K;
  int32_t G;               // K / 128
  int32_t nw;              // waves that hold K ranges
  int32_t gpw;             // groups per wave (split-K share)
  int32_t sk;              // groups per staged activation slice
  int32_t xs_stride;       // bf16 values per staged token row (a multiple of 512)
  int32_t wave_lds;        // bytes of LDS per wave
  int32_t fin_offset;      // run workgroups: LDS byte offset of the collected outputs (0: stored per tile)
  int32_t vec_scales;      // 1: eight scales per 16-byte load (tiled layout, or row-major rows
                           //    16-byte aligned with G % 8 == 0)
  int32_t tiled;           // 1: packed points at the tiled layout (scales inside it)
  int64_t tile_bytes;      // tiled layout: bytes per 16-row tile
  int32_t run_tiles;       // run workgroups: tiles per wave
  int32_t reserved;
  int64_t reserved1;       // unused (keeps the table record at 144 bytes)
  int64_t reserved2;
};

// Tiled weight layout (see include/w4a16.h): per 16-row tile, chunks of up
// to eight 128-column groups; a group is 16 rows x 64 code bytes in row
// order, and a chunk's codes are followed by 16 rows x 8 bf16 scales.
constexpr int kTileGroupBytes = 16 * 64;
constexpr int kTileChunkGroups = 8;
constexpr int kTileScaleBytes = 16 * kTileChunkGroups * 2;
constexpr int kTileChunkBytes = kTileChunkGroups * kTileGroupBytes + kTileScaleBytes;
inline int64_t tiled_tile_bytes(int64_t G) {
  return G * kTileGroupBytes + (G + kTileChunkGroups - 1) / kTileChunkGroups * kTileScaleBytes;
}

// Kernel shapes.  Dot: lanes split each row's K (v_dot2).  Split: matrix-core
// workgroup whose waves split K over the same 16-row tiles.  Shared:
// matrix-core workgroup whose waves own different tiles over all of K.  Run:
// a shared workgroup whose waves stream several whole tiles each, the load
// ring running from one tile into the next (all of K staged once).
constexpr int kDot = 1, kSplit = 2, kShared = 3, kRun = 4;
constexpr int kDotMaxT = 8;  // the dot kernel is built for T <= 8
// Run workgroups whose activations fit but leave no room for their outputs
// take K in slices, so that the outputs are still collected in LDS.
constexpr bool kSlicedRuns = true;

// Matrix-core tile choice: shape, 16-row tiles per wave, waves per workgroup.
struct Tile {
  int shape;
  int rt;
  int nw;
};

struct Plan {
  int variant;   // kDot, kSplit, kShared or kRun
  int rt;        // 16-row tiles per wave (matrix core) / rows per wave (dot)
  int threads;   // threads per workgroup
  int64_t grid;  // workgroups
  int lds;       // dynamic LDS bytes
  bool tiled;    // every problem is in the tiled layout: kernels built for it alone
  bool rowmajor; // every problem is row-major: kernels built for it alone
};

// Parse "split,rt,waves" or "shared,rt,waves" (rt 1, 2 or 4; waves 1-8, or
// 1-16 for shared workgroups of one tile per wave), or "run,tiles,waves"
// (tiles per wave 1-16, waves 1-16).
bool parse_tile(const char* text, Tile* t);
// Replaces *t by the measurement override of grouped (batch) or single
// launches, if one is set: initially from W4A16_BATCH_TILE / W4A16_TILE
// (read once per process), then by set_tile_override ("" or null: none;
// false for a spec that does not parse).
bool tile_override(bool batch, Tile* t);
bool set_tile_override(bool batch, const char* spec);

// Fill the tiling fields of `a` and return the launch plan.
Plan plan_mfma(GemvArgs& a, int T, int cus);  // default matrix-core tiling of one launch (cus: CUs of the device)
Plan plan_dot(GemvArgs& a, int T);
// tiled_kernel: the launch runs the kernels built for the tiled layout only
// (every problem tiled; one tile per wave); row_kernel: those built for the
// row-major layout only (every problem row-major); neither: the kernels
// that read either layout (a grouped launch mixing them).
// batch: planning one problem of a grouped launch (a run tile whose
// activations do not fit stays a run-kernel problem with run_tiles = 0).
Plan plan_tile(GemvArgs& a, int T, const Tile& t, bool tiled_kernel, bool row_kernel, bool batch);
// Waves of a shared workgroup of one tile per wave: 16 (one workgroup per CU,
// up to 160 KB of LDS) when T rows of K activations need more than 80 KB,
// else 4 at T = 1 and 8 above (MI355X sweeps of the tiled layout).
int shared_waves(int T, int64_t K);


hipError_t launch(const GemvArgs& a, const Plan& p, int T, hipStream_t s);
hipError_t launch_batch(const GemvArgs* table_dev, int count, const Plan& p, int T, hipStream_t s);
// Tiled layout of rows row_ids[0..N) of an n_rows-row weight (all N rows
// when row_ids is null, n_rows = N).
hipError_t launch_repack(const uint8_t* packed, const uint16_t* scales, const int32_t* row_ids, int64_t n_rows,
                         int64_t N, int32_t K, uint8_t* tiled, hipStream_t s);
hipError_t launch_argmax_final(const int2* partial, int64_t nparts, int T, int32_t* id, float* val, hipStream_t s);

// Streaming read of bytes (a multiple of 16) over `workgroups` workgroups
// of 256 threads; sink holds workgroups * 256 words.
hipError_t launch_stream_read(const void* src, int64_t bytes, unsigned* sink, int workgroups, hipStream_t s);

// Upper bound of the workgroups any plan uses for n_out rows (sizes the argmax workspace).
int64_t max_workgroups(int64_t n_out);

// Verify epilogue (w4a16_epilogue.hip).  The top-k workspace holds
// T * topk_chunks(n) * k candidate keys of 8 bytes.
int64_t topk_chunks(int64_t n);
hipError_t launch_topk(const float* scores, int64_t n, int T, const int32_t* row_ids, int k, int32_t* top_ids,
                       float* top_vals, void* workspace, hipStream_t s);
hipError_t launch_greedy(const int32_t* target, const int32_t* draft, int n_seq, int rows, int32_t* accepted,
                         int32_t* tokens, hipStream_t s);
// Draft-head id list: at most kMaxSeqIds sequence ids, vocabularies of at
// most kMaxUnionVocab ids (its bitmap lives in LDS).
constexpr int kMaxSeqIds = 4096;
constexpr int64_t kMaxUnionVocab = 524288;
hipError_t launch_draft_union(const int32_t* base, int n_base, const int32_t* seq, int n_seq, int n_rows,
                              int32_t* out, int32_t* n_out, hipStream_t s);

}  // namespace w4a16
