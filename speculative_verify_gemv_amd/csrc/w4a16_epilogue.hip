// Verify epilogue of libw4a16 (gfx950): per-row top-k of head scores and
// greedy acceptance of drafted tokens.
//
// Top-k.  The OpenJet engine page ("How it gets its speed") keeps the 32
// best logits of each verified row for its sampler; the qwen-warp article
// ("What each one calls the same answer") rescores the quantized head's 16
// best candidates.  For each activation row t of scores[T][n]: the k largest
// non-NaN scores with their vocabulary ids, score descending, equal scores
// by ascending id (entry 0 is the head's argmax).  Every candidate is one
// 64-bit key whose unsigned order is that order: an order-preserving image
// of the fp32 score (with -0 taken as +0) in the high word and 0x7fffffff -
// id in the low word; a NaN score, a negative id or a position past n is the
// key 0, below every real candidate.  Two launches: workgroups sort chunks of
// 2048 keys of one row in LDS (bitonic network) and keep their best k; one
// workgroup per row then merges those candidates, 4096 keys at a time.
//
// Greedy acceptance.  The same article section: greedy acceptance is an
// argmax equality over the verify rows; the OpenJet page ("How it works"):
// the host reads back only the accepted tokens.  One thread per sequence.
#include "w4a16_internal.h"

namespace w4a16 {
namespace {

typedef unsigned long long u64;

constexpr int kChunk = 2048;        // keys per first-stage workgroup
constexpr int kChunkThreads = 256;
constexpr int kMerge = 4096;        // keys per second-stage sort
constexpr int kMergeThreads = 1024;

__device__ __forceinline__ u64 score_key(float v, int64_t id) {
  if (__builtin_isnan(v) || id < 0 || id > 0x7fffffffLL) return 0ull;
  const unsigned b = __float_as_uint(v == 0.0f ? 0.0f : v);
  const unsigned hi = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((u64)hi << 32) | (u64)(0x7fffffffu - (unsigned)id);
}

__device__ __forceinline__ void key_decode(u64 key, int32_t& id, float& v) {
  if (key == 0ull) {
    id = -1;
    v = __builtin_nanf("");
    return;
  }
  const unsigned hi = (unsigned)(key >> 32);
  v = __uint_as_float((hi & 0x80000000u) ? (hi & 0x7fffffffu) : ~hi);
  id = (int32_t)(0x7fffffffu - (unsigned)(key & 0xffffffffu));
}

// Sorts s[0..N) (N a power of two) into descending order with all threads
// of the workgroup; ends with a barrier.
template <int N>
__device__ __forceinline__ void bitonic_desc(u64* s) {
  for (int size = 2; size <= N; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < N / 2; i += blockDim.x) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool desc = (lo & size) == 0;
        const u64 a = s[lo], b = s[hi];
        if ((a < b) == desc) {
          s[lo] = b;
          s[hi] = a;
        }
      }
      __syncthreads();
    }
  }
}

// Workgroup (chunk c, row t): the best k keys of scores[t][c*kChunk ..).
__global__ void __launch_bounds__(kChunkThreads) w4a16_topk_chunks(const float* __restrict__ scores, int64_t n,
                                                                   const int32_t* __restrict__ row_ids, int k,
                                                                   u64* __restrict__ part) {
  __shared__ u64 s[kChunk];
  const int t = blockIdx.y;
  const int64_t c = blockIdx.x, nchunks = gridDim.x;
  const int64_t base = c * kChunk;
  const float* row = scores + (int64_t)t * n;
  for (int i = threadIdx.x; i < kChunk; i += blockDim.x) {
    const int64_t pos = base + i;
    u64 key = 0ull;
    if (pos < n) key = score_key(row[pos], row_ids ? (int64_t)row_ids[pos] : pos);
    s[i] = key;
  }
  __syncthreads();
  bitonic_desc<kChunk>(s);
  for (int j = threadIdx.x; j < k; j += blockDim.x) part[((int64_t)t * nchunks + c) * k + j] = s[j];
}

// Workgroup t: the best k of the m candidate keys of row t, merged kMerge at
// a time (the running best stays in the first k slots).
__global__ void __launch_bounds__(kMergeThreads) w4a16_topk_merge(const u64* __restrict__ part, int64_t m, int k,
                                                                  int32_t* __restrict__ top_ids,
                                                                  float* __restrict__ top_vals) {
  __shared__ u64 s[kMerge];
  const int t = blockIdx.x;
  const u64* cand = part + (int64_t)t * m;
  for (int i = threadIdx.x; i < k; i += blockDim.x) s[i] = 0ull;
  for (int64_t b = 0; b < m || b == 0; b += kMerge - k) {
    for (int i = k + threadIdx.x; i < kMerge; i += blockDim.x) {
      const int64_t j = b + (i - k);
      s[i] = j < m ? cand[j] : 0ull;
    }
    __syncthreads();
    bitonic_desc<kMerge>(s);
    if (b + (kMerge - k) >= m) break;
  }
  for (int j = threadIdx.x; j < k; j += blockDim.x) {
    int32_t id;
    float v;
    key_decode(s[j], id, v);
    top_ids[(int64_t)t * k + j] = id;
    if (top_vals) top_vals[(int64_t)t * k + j] = v;
  }
}

__global__ void __launch_bounds__(64) w4a16_greedy(const int32_t* __restrict__ target,
                                                   const int32_t* __restrict__ draft, int n_seq, int rows,
                                                   int32_t* __restrict__ accepted, int32_t* __restrict__ tokens) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= n_seq) return;
  const int32_t* tg = target + (int64_t)s * rows;
  const int32_t* dr = draft + (int64_t)s * (rows - 1);
  int a = 0;
  while (a < rows - 1 && tg[a] >= 0 && tg[a] == dr[a]) ++a;
  accepted[s] = a;
  if (tokens)
    for (int r = 0; r < rows; ++r) tokens[(int64_t)s * rows + r] = r <= a ? tg[r] : -1;
}

}  // namespace

int64_t topk_chunks(int64_t n) { return (n + kChunk - 1) / kChunk; }

hipError_t launch_topk(const float* scores, int64_t n, int T, const int32_t* row_ids, int k, int32_t* top_ids,
                       float* top_vals, void* workspace, hipStream_t s) {
  const int64_t nchunks = topk_chunks(n);
  u64* part = static_cast<u64*>(workspace);
  hipLaunchKernelGGL(w4a16_topk_chunks, dim3((unsigned)nchunks, (unsigned)T), dim3(kChunkThreads), 0, s, scores, n,
                     row_ids, k, part);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  hipLaunchKernelGGL(w4a16_topk_merge, dim3((unsigned)T), dim3(kMergeThreads), 0, s, part, nchunks * k, k, top_ids,
                     top_vals);
  return hipGetLastError();
}

hipError_t launch_greedy(const int32_t* target, const int32_t* draft, int n_seq, int rows, int32_t* accepted,
                         int32_t* tokens, hipStream_t s) {
  hipLaunchKernelGGL(w4a16_greedy, dim3((unsigned)((n_seq + 63) / 64)), dim3(64), 0, s, target, draft, n_seq, rows,
                     accepted, tokens);
  return hipGetLastError();
}

}  // namespace w4a16
