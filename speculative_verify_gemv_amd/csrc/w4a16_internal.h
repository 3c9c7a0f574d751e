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
  int32_t xs_stride;       // halves per staged token row
  int32_t wave_lds;        // bytes of LDS per wave
  int32_t fin_offset;      // byte offset of the final-value area
  int32_t vec_scales;      // 1: scale rows are 16-byte aligned and G % 8 == 0 (8 scales per load)
  int32_t reserved;
};

struct Plan {
  int variant;   // 1 dot, 2 mfma (split-K), 3 mfma (streaming)
  int rt;        // 16-row tiles per workgroup (mfma) / rows per wave (dot)
  int pd;        // groups of weight loads in flight per wave (mfma)
  int threads;   // threads per workgroup
  int64_t grid;  // workgroups
  int lds;       // dynamic LDS bytes
};

// Fill the tiling fields of `a` and return the launch plan.
Plan plan_mfma(GemvArgs& a, int T);
Plan plan_dot(GemvArgs& a, int T);
// Tiling of one problem of a grouped launch whose rt, pd and wave count are fixed.
void plan_mfma_fixed(GemvArgs& a, int T, int rt, int pd, int nw, int* lds, int64_t* grid);
void plan_stream(GemvArgs& a, int T, int pd, int nwv, int* lds, int64_t* grid);

hipError_t launch(const GemvArgs& a, const Plan& p, int T, hipStream_t s);
hipError_t launch_batch(const GemvArgs* table_dev, int count, const Plan& p, int T, hipStream_t s);
hipError_t launch_argmax_final(const int2* partial, int64_t nparts, int T, int32_t* id, float* val, hipStream_t s);

// Upper bound of the workgroups any plan uses for n_out rows (sizes the argmax workspace).
int64_t max_workgroups(int64_t n_out);

}  // namespace w4a16
