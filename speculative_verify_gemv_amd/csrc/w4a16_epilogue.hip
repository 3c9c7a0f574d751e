// Verify epilogue of libw4a16 (gfx950): per-row top-k of head scores and
// greedy acceptance of drafted tokens.
//
// Top-k.  The OpenJet engine page ("How it gets its speed") hands its
// sampler the highest 32 scores of every verified row; the qwen-warp article
// ("What each one calls the same answer") rescores the 16 highest
// candidates of the quantized head.  For each activation row t of scores[T][n]: the k largest
// non-NaN scores with their vocabulary ids, score descending, equal scores
// by ascending id (entry 0 is the head's argmax).  Every candidate is one
// 64-bit key whose unsigned order is that order: an order-preserving image
// of the fp32 score (with -0 taken as +0) in the high word and 0x7fffffff -
// id in the low word; a NaN score, a negative id or a position past n is the
// key 0, below every real candidate.  Two launches: workgroups sort chunks of
// 2048 keys of one row and keep their best k, one workgroup per row then
// merges those lists.  Both bound the k-th largest key from below by the
// k-th largest of part maxima, rank the few keys at or above the bound by
// counting, and fall back to a bitonic sort in LDS when many keys tie.
//
// Greedy acceptance.  The same article section: under greedy decoding a
// draft is kept when it equals the target's argmax on its verify row; the
// OpenJet page ("How it works"): only the accepted tokens travel to the
// host.  One thread per sequence.
//
// Draft-head id list.  The OpenJet page ("How it gets its speed"): the
// drafter's head scores a fixed list of 32,768 common tokens, extended at
// run time by whichever ids of the current sequence the list lacks.  One workgroup: the base
// ids go into a vocabulary bitmap in LDS; an LDS hash table keeps the first
// position of every sequence id (atomic insert, atomic minimum); a prefix
// count over positions then places the new ids in order of first
// appearance after the base list.
#include "w4a16_internal.h"

namespace w4a16 {
namespace {

typedef unsigned long long u64;

constexpr int kChunk = 2048;        // keys per first-stage workgroup
constexpr int kChunkThreads = 256;
constexpr int kMerge = 4096;        // keys per second-stage sort
constexpr int kMergeThreads = 256;

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

// One compare-exchange of the bitonic network: element lo of a block that
// runs descending (desc) or ascending, against element lo + stride.
__device__ __forceinline__ void cas(u64& a, u64& b, bool desc) {
  const bool swap = desc ? (a < b) : (a > b);
  const u64 lo = swap ? b : a, hi = swap ? a : b;
  a = lo;
  b = hi;
}

// LDS slot of sort position i: bits 0-4 XORed with bits 5-9, so that the E
// consecutive positions of each thread (register passes) and the pairs of
// consecutive threads (LDS passes) fall into different banks.
__device__ __forceinline__ int slot(int i) { return i ^ ((i >> 5) & 31); }

// Sorts the N keys at positions 0..N-1 (N a power of two, position i in LDS
// slot slot(i); arrange them that way, e.g. by writing key i to s[slot(i)])
// into descending (DESC) or ascending order with NT threads (the whole
// workgroup); each thread owns the E = N / NT consecutive positions from
// threadIdx.x * E.  Passes whose stride is below E run on the thread's own
// keys in registers; the wider passes go through LDS, each thread loading
// all its pairs before it compares and stores them.  Ends with a barrier.
template <int N, int NT, bool DESC = true>
__device__ __forceinline__ void bitonic_sort(u64* s) {
  constexpr int E = N / NT;
  static_assert(E >= 2 && (E & (E - 1)) == 0 && N % NT == 0 && N >= 1024, "E a power of two >= 2, N >= 1024");
  const int t0 = threadIdx.x * E;
  u64 v[E];
#pragma unroll
  for (int j = 0; j < E; ++j) v[j] = s[slot(t0 + j)];
  // blocks of up to E keys: all in registers
#pragma unroll
  for (int size = 2; size <= E; size <<= 1)
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1)
#pragma unroll
      for (int j = 0; j < E; ++j)
        if ((j & stride) == 0) cas(v[j], v[j + stride], (((t0 + j) & size) == 0) == DESC);
#pragma unroll
  for (int j = 0; j < E; ++j) s[slot(t0 + j)] = v[j];
  __syncthreads();
  for (int size = 2 * E; size <= N; size <<= 1) {
    for (int stride = size >> 1; stride >= E; stride >>= 1) {
      u64 a[E / 2], b[E / 2];
      int lo[E / 2];
#pragma unroll
      for (int q = 0; q < E / 2; ++q) {
        const int i = threadIdx.x + q * NT;
        lo[q] = 2 * i - (i & (stride - 1));
        a[q] = s[slot(lo[q])];
        b[q] = s[slot(lo[q] + stride)];
      }
#pragma unroll
      for (int q = 0; q < E / 2; ++q) {
        cas(a[q], b[q], ((lo[q] & size) == 0) == DESC);
        s[slot(lo[q])] = a[q];
        s[slot(lo[q] + stride)] = b[q];
      }
      __syncthreads();
    }
#pragma unroll
    for (int j = 0; j < E; ++j) v[j] = s[slot(t0 + j)];
#pragma unroll
    for (int stride = E >> 1; stride > 0; stride >>= 1)
#pragma unroll
      for (int j = 0; j < E; ++j)
        if ((j & stride) == 0) cas(v[j], v[j + stride], (((t0 + j) & size) == 0) == DESC);
#pragma unroll
    for (int j = 0; j < E; ++j) s[slot(t0 + j)] = v[j];
    __syncthreads();
  }
}

// Ranks by counting: for the m keys c[0..m) (in LDS), key i goes to output
// slot (number of larger keys + number of equal keys before it), which is a
// permutation of 0..m-1 in descending order; keys of rank < k are passed to
// put(rank, key).  m * m / threads compares.
template <typename Put>
__device__ __forceinline__ void rank_top(const u64* c, int m, int k, Put put) {
  for (int i = threadIdx.x; i < m; i += blockDim.x) {
    const u64 v = c[i];
    int r = 0;
    for (int j = 0; j < m; ++j) {
      const u64 o = c[j];
      r += (o > v || (o == v && j < i)) ? 1 : 0;
    }
    if (r < k) put(r, v);
  }
}

// Lower bound for the k-th largest key of a set split into parts: the k-th
// largest of the parts' maxima (there are k keys at least that large).  mx
// is this thread's part maximum, all[0..nparts) every part's; ties count
// the lower part first.  Returns the bound on the thread whose maximum has
// rank k-1, else 0 (the caller publishes it through LDS).
__device__ __forceinline__ u64 kth_of_maxima(const u64* all, int nparts, int part, u64 mx, int k) {
  int r = 0;
  for (int j = 0; j < nparts; ++j) {
    const u64 o = all[j];
    r += (o > mx || (o == mx && j < part)) ? 1 : 0;
  }
  return r == k - 1 ? mx : 0ull;
}

constexpr int kCand = 512;  // candidates ranked by counting; more go to the full sort

// Workgroup (chunk c, row t): the best k keys of scores[t][c*kChunk ..) in
// descending order (zero keys past the chunk's countable entries).  Each
// thread holds 8 keys; the k-th largest thread maximum bounds the chunk's
// k-th largest key from below, so only keys at or above it (a few dozen on
// real scores) are ranked; a chunk with more (many equal keys) is sorted.
__global__ void __launch_bounds__(kChunkThreads) w4a16_topk_chunks(const float* __restrict__ scores, int64_t n,
                                                                   const int32_t* __restrict__ row_ids, int k,
                                                                   u64* __restrict__ part) {
  constexpr int E = kChunk / kChunkThreads;
  __shared__ u64 s[kChunk];
  __shared__ u64 tmax[kChunkThreads];
  __shared__ u64 bound;
  __shared__ int count;
  const int t = blockIdx.y, tid = threadIdx.x;
  const int64_t c = blockIdx.x, nchunks = gridDim.x;
  const int64_t base = c * kChunk;
  const float* row = scores + (int64_t)t * n;
  u64 key[E], mx = 0ull;
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const int64_t pos = base + tid + j * kChunkThreads;
    key[j] = pos < n ? score_key(row[pos], row_ids ? (int64_t)row_ids[pos] : pos) : 0ull;
    mx = key[j] > mx ? key[j] : mx;
  }
  tmax[tid] = mx;
  if (tid == 0) {
    count = 0;
    bound = 0ull;
  }
  __syncthreads();
  const u64 b = kth_of_maxima(tmax, kChunkThreads, tid, mx, k);
  if (b != 0ull) bound = b;
  __syncthreads();
  const u64 th = bound;
#pragma unroll
  for (int j = 0; j < E; ++j)
    if (key[j] != 0ull && key[j] >= th) {
      const int at = atomicAdd(&count, 1);
      if (at < kCand) s[at] = key[j];
    }
  __syncthreads();
  const int m = count;
  u64* out = part + (t * nchunks + c) * k;
  if (m <= kCand) {
    rank_top(s, m, k, [&](int r, u64 v) { out[r] = v; });
    for (int i = m + tid; i < k; i += kChunkThreads) out[i] = 0ull;
    return;
  }
  __syncthreads();  // every thread is done with the candidate list
#pragma unroll
  for (int j = 0; j < E; ++j) s[slot(tid + j * kChunkThreads)] = key[j];
  __syncthreads();
  bitonic_sort<kChunk, kChunkThreads>(s);
  for (int j = tid; j < k; j += kChunkThreads) out[j] = s[slot(j)];
}

constexpr int kHeads = 1024;  // chunk lists whose heads bound the row's k-th key

// Workgroup t: the best k of the row's chunk lists (nchunks lists of k keys,
// each descending).  The k-th largest list head bounds the row's k-th key
// from below, so only keys at or above it are ranked; with more chunks than
// kHeads or more survivors than kCand, all candidates are merged by sorting
// kMerge at a time (the running best in the first k slots).
__global__ void __launch_bounds__(kMergeThreads) w4a16_topk_merge(const u64* __restrict__ part, int64_t nchunks,
                                                                  int k, int32_t* __restrict__ top_ids,
                                                                  float* __restrict__ top_vals) {
  __shared__ u64 s[kMerge];
  __shared__ u64 heads[kHeads];
  __shared__ u64 bound;
  __shared__ int count;
  const int t = blockIdx.x, tid = threadIdx.x;
  const int64_t m = nchunks * k;
  const u64* cand = part + (int64_t)t * m;
  auto emit = [&](int j, u64 key) {
    int32_t id;
    float v;
    key_decode(key, id, v);
    top_ids[(int64_t)t * k + j] = id;
    if (top_vals) top_vals[(int64_t)t * k + j] = v;
  };
  if (nchunks <= kHeads) {
    for (int c = tid; c < nchunks; c += kMergeThreads) heads[c] = cand[(int64_t)c * k];
    if (tid == 0) {
      count = 0;
      bound = 0ull;
    }
    __syncthreads();
    for (int c = tid; c < nchunks; c += kMergeThreads) {
      const u64 b = kth_of_maxima(heads, (int)nchunks, c, heads[c], k);
      if (b != 0ull) bound = b;
    }
    __syncthreads();
    const u64 th = bound;
    constexpr int kBatch = 8;  // candidate loads in flight per thread
    for (int64_t b0 = 0; b0 < m; b0 += (int64_t)kBatch * kMergeThreads) {
      u64 key[kBatch];
#pragma unroll
      for (int q = 0; q < kBatch; ++q) {
        const int64_t i = b0 + tid + (int64_t)q * kMergeThreads;
        key[q] = i < m ? cand[i] : 0ull;
      }
#pragma unroll
      for (int q = 0; q < kBatch; ++q)
        if (key[q] != 0ull && key[q] >= th) {
          const int at = atomicAdd(&count, 1);
          if (at < kCand) s[at] = key[q];
        }
    }
    __syncthreads();
    const int cnt = count;
    if (cnt <= kCand) {
      rank_top(s, cnt, k, emit);
      for (int i = cnt + tid; i < k; i += kMergeThreads) emit(i, 0ull);
      return;
    }
    __syncthreads();  // every thread is done with the candidate list
  }
  for (int i = tid; i < k; i += kMergeThreads) s[slot(i)] = 0ull;
  for (int64_t b = 0; b < m || b == 0; b += kMerge - k) {
    for (int i = k + tid; i < kMerge; i += kMergeThreads) {
      const int64_t j = b + (i - k);
      s[slot(i)] = j < m ? cand[j] : 0ull;
    }
    __syncthreads();
    bitonic_sort<kMerge, kMergeThreads>(s);
    if (b + (kMerge - k) >= m) break;
  }
  for (int j = tid; j < k; j += kMergeThreads) emit(j, s[slot(j)]);
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
constexpr int kHashSlots = 2 * kMaxSeqIds;  // open addressing, load factor <= 1/2

// LDS of the union kernel: the vocabulary bitmap, then the hash table's ids
// (id + 1, 0 = empty) and first positions, then one mark per sequence
// position (the id it adds, or -1), then the wave sums of the prefix count.
__host__ __device__ constexpr int union_table_offset(int64_t n_rows) {
  return (int)((((n_rows + 31) / 32) * 4 + 15) / 16 * 16);
}
__host__ __device__ constexpr int union_lds(int64_t n_rows) {
  return union_table_offset(n_rows) + kHashSlots * 8 + kMaxSeqIds * 4 + (kUnionThreads / 64 + 1) * 4;
}

__device__ __forceinline__ int hash_slot(unsigned id) { return (int)((id * 2654435761u) >> 19) & (kHashSlots - 1); }

__global__ void __launch_bounds__(kUnionThreads) w4a16_draft_union(const int32_t* __restrict__ base, int n_base,
                                                                   const int32_t* __restrict__ seq, int n_seq,
                                                                   int n_rows, int32_t* __restrict__ out,
                                                                   int32_t* __restrict__ n_out) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  unsigned* bits = reinterpret_cast<unsigned*>(smem);
  unsigned* tab_id = reinterpret_cast<unsigned*>(smem + union_table_offset(n_rows));
  int* tab_pos = reinterpret_cast<int*>(tab_id + kHashSlots);
  int32_t* mark = tab_pos + kHashSlots;
  int* wsum = mark + kMaxSeqIds;
  const int tid = threadIdx.x, nt = blockDim.x;
  const int words = (n_rows + 31) >> 5;
  for (int i = tid; i < words; i += nt) bits[i] = 0u;
  for (int i = tid; i < kHashSlots; i += nt) {
    tab_id[i] = 0u;
    tab_pos[i] = 0x7fffffff;
  }
  for (int i = tid; i < kMaxSeqIds; i += nt) mark[i] = -1;
  __syncthreads();
  // the base list, verbatim, and its in-range ids in the bitmap (8 loads in
  // flight per thread)
  for (int b0 = 0; b0 < n_base; b0 += 8 * nt) {
    int32_t id[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int i = b0 + tid + q * nt;
      id[q] = i < n_base ? base[i] : -1;
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int i = b0 + tid + q * nt;
      if (i >= n_base) continue;
      out[i] = id[q];
      if (id[q] >= 0 && id[q] < n_rows) atomicOr(&bits[id[q] >> 5], 1u << (id[q] & 31));
    }
  }
  // first position of every in-range sequence id (at most kMaxSeqIds ids in
  // twice as many slots, so a probe always ends)
  for (int i = tid; i < n_seq; i += nt) {
    const int32_t id = seq[i];
    if (id < 0 || id >= n_rows) continue;
    const unsigned key = (unsigned)id + 1u;
    for (int h = hash_slot((unsigned)id);; h = (h + 1) & (kHashSlots - 1)) {
      const unsigned old = atomicCAS(&tab_id[h], 0u, key);
      if (old == 0u || old == key) {
        atomicMin(&tab_pos[h], i);
        break;
      }
    }
  }
  __syncthreads();
  // a position adds its id if it is the id's first position and the base
  // list does not hold the id
  for (int i = tid; i < n_seq; i += nt) {
    const int32_t id = seq[i];
    if (id < 0 || id >= n_rows || ((bits[id >> 5] >> (id & 31)) & 1u)) continue;
    const unsigned key = (unsigned)id + 1u;
    int h = hash_slot((unsigned)id);
    while (tab_id[h] != key) h = (h + 1) & (kHashSlots - 1);
    if (tab_pos[h] == i) mark[i] = id;
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
  hipLaunchKernelGGL(w4a16_topk_merge, dim3((unsigned)T), dim3(kMergeThreads), 0, s, part, nchunks, k, top_ids,
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
