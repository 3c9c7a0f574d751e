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
//
// Draft-head id list.  The OpenJet page ("How it gets its speed"): the draft
// head covers the 32,768 most frequent tokens plus the tokens of the current
// sequence missing from them, added on the fly.  One workgroup: the base
// ids go into a vocabulary bitmap in LDS; the sequence's (id, position)
// pairs are sorted in LDS so that the first appearance of each id is the
// first of its run; a prefix count over positions then places the new ids
// in order of first appearance after the base list.
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

// Sorts s[0..N) (N a power of two) into descending (DESC) or ascending
// order with all threads of the workgroup; ends with a barrier.
template <int N, bool DESC = true>
__device__ __forceinline__ void bitonic_sort(u64* s) {
  for (int size = 2; size <= N; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < N / 2; i += blockDim.x) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool desc = ((lo & size) == 0) == DESC;  // this pair's block runs descending
        const u64 a = s[lo], b = s[hi];
        if (desc ? (a < b) : (a > b)) {
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
  bitonic_sort<kChunk>(s);
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
    bitonic_sort<kMerge>(s);
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

constexpr int kUnionThreads = 1024;

// LDS of the union kernel: the vocabulary bitmap, then kMaxSeqIds sort keys,
// then kMaxSeqIds marks (the id a position adds, or -1), then the wave sums.
__host__ __device__ constexpr int union_keys_offset(int64_t n_rows) {
  return (int)((((n_rows + 31) / 32) * 4 + 15) / 16 * 16);
}
__host__ __device__ constexpr int union_lds(int64_t n_rows) {
  return union_keys_offset(n_rows) + kMaxSeqIds * 8 + kMaxSeqIds * 4 + (kUnionThreads / 64 + 1) * 4;
}

__global__ void __launch_bounds__(kUnionThreads) w4a16_draft_union(const int32_t* __restrict__ base, int n_base,
                                                                   const int32_t* __restrict__ seq, int n_seq,
                                                                   int n_rows, int32_t* __restrict__ out,
                                                                   int32_t* __restrict__ n_out) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  unsigned* bits = reinterpret_cast<unsigned*>(smem);
  u64* keys = reinterpret_cast<u64*>(smem + union_keys_offset(n_rows));
  int32_t* mark = reinterpret_cast<int32_t*>(keys + kMaxSeqIds);
  int* wsum = reinterpret_cast<int*>(mark + kMaxSeqIds);
  const int tid = threadIdx.x, nt = blockDim.x;
  const int words = (n_rows + 31) >> 5;
  for (int i = tid; i < words; i += nt) bits[i] = 0u;
  __syncthreads();
  // the base list, verbatim, and its in-range ids in the bitmap
  for (int i = tid; i < n_base; i += nt) {
    const int32_t id = base[i];
    out[i] = id;
    if (id >= 0 && id < n_rows) atomicOr(&bits[id >> 5], 1u << (id & 31));
  }
  // (id, position) of every in-range sequence id; the rest sort to the end
  for (int i = tid; i < kMaxSeqIds; i += nt) {
    u64 key = ~0ull;
    if (i < n_seq) {
      const int32_t id = seq[i];
      if (id >= 0 && id < n_rows) key = ((u64)(unsigned)id << 32) | (unsigned)i;
    }
    keys[i] = key;
    mark[i] = -1;
  }
  __syncthreads();
  bitonic_sort<kMaxSeqIds, false>(keys);
  // the first position of each id adds it unless the base list has it
  for (int j = tid; j < kMaxSeqIds; j += nt) {
    const u64 key = keys[j];
    if (key == ~0ull) continue;
    const unsigned id = (unsigned)(key >> 32);
    const bool first = j == 0 || (unsigned)(keys[j - 1] >> 32) != id;
    if (first && !((bits[id >> 5] >> (id & 31)) & 1u)) mark[(unsigned)(key & 0xffffffffu)] = (int32_t)id;
  }
  __syncthreads();
  // prefix count of the adding positions, in position order
  constexpr int kPer = kMaxSeqIds / kUnionThreads;
  int c = 0;
#pragma unroll
  for (int q = 0; q < kPer; ++q) c += mark[tid * kPer + q] >= 0 ? 1 : 0;
  const int lane = tid & 63, wave = tid >> 6;
  int incl = c;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off);
    if (lane >= off) incl += v;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int w = 0; w < nt / 64; ++w) {
      const int v = wsum[w];
      wsum[w] = run;
      run += v;
    }
    wsum[nt / 64] = run;
  }
  __syncthreads();
  int at = n_base + wsum[wave] + incl - c;
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int32_t id = mark[tid * kPer + q];
    if (id >= 0) out[at++] = id;
  }
  const int total = n_base + wsum[nt / 64];
  for (int i = total + tid; i < n_base + n_seq; i += nt) out[i] = -1;
  if (tid == 0) *n_out = total;
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

namespace w4a16 {

hipError_t launch_draft_union(const int32_t* base, int n_base, const int32_t* seq, int n_seq, int n_rows,
                              int32_t* out, int32_t* n_out, hipStream_t s) {
  const int lds = union_lds(n_rows);
  if (lds > 65536) {  // above 64 KB of dynamic LDS the kernel has to opt in
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&w4a16_draft_union),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(w4a16_draft_union, dim3(1), dim3(kUnionThreads), lds, s, base, n_base, seq, n_seq, n_rows, out,
                     n_out);
  return hipGetLastError();
}

}  // namespace w4a16
