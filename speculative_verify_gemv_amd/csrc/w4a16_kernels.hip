// W4A16 skinny matmul kernels for AMD Instinct MI355X (gfx950, CDNA4).
//
// y[t][n] = sum_k (q[n][k] - 8) * scale[n][k/128] * x[t][k]   (fp32 out)
//
// The weight format -- little-endian words of eight nibbles, level = nibble
// minus 8, one bf16 scale per 128 columns applied after the group's sum -- is
// the one the qwen-warp/llamAmpere article gives under "qwen-warp: keep the
// activations in bf16".  That engine turns a nibble pair into exact bf16
// levels with one OR and one packed bf16 FMA; gfx950 has no packed bf16 add
// or FMA, so here the exact levels are formed in fp16 instead:
//
//   (w & 0x000F000F) | 0x6400_6400  is the fp16 pair (1024 + q0, 1024 + q4)
//   (w & 0x00F000F0) | 0x5400_5400  is the fp16 pair (  64 + q1,   64 + q5)
//
// (at 1024 the fp16 spacing is 1, at 64 it is 1/16 and the nibble sits four
// bits higher), and one v_pk_add_f16 with -1032 / -72 gives (q - 8) exactly.
// A 32-bit word of codes becomes eight exact fp16 levels in the slot order
// k+0, k+4, k+1, k+5, k+2, k+6, k+3, k+7 with 9 VALU operations.
//
// Activations are converted once per workgroup slice to fp16 in the same
// slot order, scaled by 2^E (E chosen per token row and slice from the
// largest |x|), so every bf16 value that matters is represented exactly; the
// power of two is removed again when the slice's partial sums are folded, so
// the result equals the unscaled fp32 arithmetic.  Every product (q-8)*x is
// exact in fp32; sums are fp32.
//
// Two variants:
//  * mfma: tokens are the A operand of v_mfma_f32_16x16x32_f16 (T padded to
//    16 rows with zeros), weights the B operand (16 output rows x 32 k).  A
//    lane owns one output row and a quarter of each 128-column group, loads
//    its 16 bytes of that group with one nontemporal 128-bit load, and feeds
//    the four words to four MFMAs.  Each 128-column group gets a fresh
//    accumulator that is then scaled in fp32.  The waves of a workgroup split
//    K; their partials are summed through LDS in wave order.
//  * dot: lanes split a row's K in 16-byte chunks; v_dot2_f32_f16 forms each
//    chunk's partial, which is scaled by its group scale; lanes are reduced
//    with a butterfly across the wavefront.
//
// Both reduce in an order fixed by (K, tiling) only, so results are
// deterministic, and identical weight rows give identical outputs.
#include <math.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <type_traits>

#include "w4a16_internal.h"

namespace w4a16 {
namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef __fp16 h8_t __attribute__((ext_vector_type(8)));  // the MFMA builtin's operand type
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef unsigned u4_t __attribute__((ext_vector_type(4)));
typedef unsigned short us2_t __attribute__((ext_vector_type(2)));

constexpr int kGroup = 128;
constexpr int kLdsCap = 65536;  // dynamic LDS per workgroup
// s_waitcnt immediate (gfx9 encoding) waiting for vmcnt = 0 only.
constexpr int kWaitVmcnt0 = 0x0F70;

__device__ __forceinline__ float bf16_to_f32(unsigned short b) { return __uint_as_float((unsigned)b << 16); }

template <typename V>
__device__ __forceinline__ unsigned as_u32(V h) {
  static_assert(sizeof(V) == 4, "packed pair");
  return __builtin_bit_cast(unsigned, h);
}

// (w & m) | c in one VALU operation (v_and_or_b32: one SGPR operand, one VGPR).
__device__ __forceinline__ unsigned and_or(unsigned w, unsigned m, unsigned c) {
  unsigned r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(w), "s"(m), "v"(c));
  return r;
}

// Eight exact fp16 levels (q - 8) of one word, slot order 0,4,1,5,2,6,3,7.
__device__ __forceinline__ u4_t levels8(unsigned w) {
  const unsigned w8 = w >> 8;
  const h2_t lo_bias = {(_Float16)-1032.0f, (_Float16)-1032.0f};
  const h2_t hi_bias = {(_Float16)-72.0f, (_Float16)-72.0f};
  const h2_t a = __builtin_bit_cast(h2_t, and_or(w, 0x000F000Fu, 0x64006400u)) + lo_bias;
  const h2_t b = __builtin_bit_cast(h2_t, and_or(w, 0x00F000F0u, 0x54005400u)) + hi_bias;
  const h2_t c = __builtin_bit_cast(h2_t, and_or(w8, 0x000F000Fu, 0x64006400u)) + lo_bias;
  const h2_t d = __builtin_bit_cast(h2_t, and_or(w8, 0x00F000F0u, 0x54005400u)) + hi_bias;
  return u4_t{as_u32(a), as_u32(b), as_u32(c), as_u32(d)};
}

// Largest bf16 magnitude (bit pattern) among the eight values of v.
__device__ __forceinline__ unsigned absmax8(u4_t v) {
  us2_t m = __builtin_bit_cast(us2_t, v.x & 0x7FFF7FFFu);
  m = __builtin_elementwise_max(m, __builtin_bit_cast(us2_t, v.y & 0x7FFF7FFFu));
  m = __builtin_elementwise_max(m, __builtin_bit_cast(us2_t, v.z & 0x7FFF7FFFu));
  m = __builtin_elementwise_max(m, __builtin_bit_cast(us2_t, v.w & 0x7FFF7FFFu));
  return max((unsigned)m.x, (unsigned)m.y);
}

__device__ __forceinline__ unsigned wave_max(unsigned m) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (unsigned)__shfl_xor((int)m, off));
  return m;
}

// Power-of-two exponent E that maps the largest |x| (bf16 magnitude bits)
// into [2^14, 2^15): every bf16 within 2^-28 of the maximum is then an exact
// fp16 normal.  0 for an all-zero or non-finite slice.
__device__ __forceinline__ int slice_exponent(unsigned mag) {
  const int e = (int)(mag >> 7);
  if (mag == 0 || e == 255) return 0;
  const int unbiased = (e == 0) ? -127 : e - 127;
  return 14 - unbiased;
}

// Eight bf16 (natural order) -> eight fp16 scaled by 2^E in slot order.
__device__ __forceinline__ u4_t convert8(u4_t v, int E) {
  const float x0 = ldexpf(__uint_as_float(v.x << 16), E), x1 = ldexpf(__uint_as_float(v.x & 0xFFFF0000u), E);
  const float x2 = ldexpf(__uint_as_float(v.y << 16), E), x3 = ldexpf(__uint_as_float(v.y & 0xFFFF0000u), E);
  const float x4 = ldexpf(__uint_as_float(v.z << 16), E), x5 = ldexpf(__uint_as_float(v.z & 0xFFFF0000u), E);
  const float x6 = ldexpf(__uint_as_float(v.w << 16), E), x7 = ldexpf(__uint_as_float(v.w & 0xFFFF0000u), E);
  return u4_t{as_u32(__builtin_amdgcn_cvt_pkrtz(x0, x4)), as_u32(__builtin_amdgcn_cvt_pkrtz(x1, x5)),
              as_u32(__builtin_amdgcn_cvt_pkrtz(x2, x6)), as_u32(__builtin_amdgcn_cvt_pkrtz(x3, x7))};
}

// v_dot2_f32_f16 on two words of packed fp16 pairs: c + a.lo*b.lo + a.hi*b.hi.
__device__ __forceinline__ float dot2(unsigned a, unsigned b, float c) {
  typedef __fp16 fp16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(fp16x2_t, a), __builtin_bit_cast(fp16x2_t, b), c, false);
}

__device__ __forceinline__ void lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Argmax candidate order: a valid id beats an invalid one; larger value wins;
// equal values go to the lower id.
__device__ __forceinline__ bool better(float v1, int i1, float v2, int i2) {
  return i1 >= 0 && (i2 < 0 || v1 > v2 || (v1 == v2 && i1 < i2));
}

__device__ __forceinline__ void wave_argmax(float& v, int& id) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ov = __shfl_xor(v, off);
    const int oi = __shfl_xor(id, off);
    if (better(ov, oi, v, id)) {
      v = ov;
      id = oi;
    }
  }
}

// Vocabulary id of output row o, or -1 if o is past the end or its id is out of range.
__device__ __forceinline__ int64_t weight_row(const GemvArgs& a, int64_t o) {
  if (o >= a.n_out) return -1;
  const int64_t w = a.row_ids ? (int64_t)a.row_ids[o] : o;
  return (w < 0 || w >= a.n_rows) ? -1 : w;
}

// Writes the per-workgroup argmax partial for token rows 0..TT-1 from the
// final values fin[(rt*TT + t)*16 + r] of rows row0 + rt*16 + r (rows < nrows).
template <int TT>
__device__ __forceinline__ void workgroup_argmax(const GemvArgs& a, const float* fin, int64_t row0, int nrows,
                                                 int lane, int64_t wg) {
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    float bv = __builtin_nanf("");
    int bi = -1;
    for (int r = lane; r < nrows; r += 64) {
      const int64_t o = row0 + r;
      const int64_t w = weight_row(a, o);
      const float v = fin[((r >> 4) * TT + t) * 16 + (r & 15)];
      if (w >= 0 && !__builtin_isnan(v) && better(v, (int)w, bv, bi)) {
        bv = v;
        bi = (int)w;
      }
    }
    wave_argmax(bv, bi);
    if (lane == 0) a.partial[wg * TT + t] = int2{__float_as_int(bv), bi};
  }
}

// ---------------------------------------------------------------- mfma ----

// Stages x[t][gs*128 .. ge*128) of all TT token rows into this wave's LDS
// area as scaled fp16 in slot order; E[t] receives each row's exponent.
template <int TT>
__device__ __forceinline__ void stage_wave(const GemvArgs& a, _Float16* xs, int gs, int ge, int lane, int (&E)[TT]) {
  const int n8 = (ge - gs) * (kGroup / 8);
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    const u4_t* src = reinterpret_cast<const u4_t*>(a.x + (int64_t)t * a.K + (int64_t)gs * kGroup);
    unsigned m = 0;
    for (int b = lane; b < n8; b += 64) m = max(m, absmax8(src[b]));
    E[t] = slice_exponent(wave_max(m));
    u4_t* dst = reinterpret_cast<u4_t*>(xs + t * a.xs_stride);
    for (int b = lane; b < n8; b += 64) dst[b] = convert8(src[b], E[t]);
  }
}

template <int TT, int RT>
__device__ __forceinline__ void fold_slice(float (&acc)[RT][4], float (&accs)[RT][4], const int (&E)[TT], int kq) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = kq * 4 + r;
    int e = E[0];
#pragma unroll
    for (int i = 1; i < TT; ++i) e = (t == i) ? E[i] : e;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      acc[rt][r] += ldexpf(accs[rt][r], -e);
      accs[rt][r] = 0.0f;
    }
  }
}

// One workgroup of the mfma variant: output rows [wg*RT*16, +RT*16) of problem
// `a`, K split over a.nw waves in ranges of a.gpw groups.  Each wave keeps PD
// groups of weight loads in flight in a register ring; the body of the
// streaming loop is straight-line so every wait names exactly the group it
// needs.  Loads past the wave's last group re-read that group and are masked
// by a zero scale.
template <int TT, int RT, int PD>
__device__ __forceinline__ void mfma_workgroup(const GemvArgs& a, int64_t wg, unsigned char* smem) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar control flow
  const int r16 = lane & 15;  // output row of the B operand / token row of the A operand
  const int kq = lane >> 4;   // quarter of the 128-column group
  const int trow = min(r16, TT - 1);  // A rows >= TT only feed D rows that are never read
  const int64_t row0 = wg * (RT * 16);
  const int64_t kh = a.K >> 1;

  const int g_begin = wave * a.gpw;
  const int n = (wave < a.nw) ? min(a.G - g_begin, a.gpw) : 0;  // wave-uniform

  float acc[RT][4];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[rt][r] = 0.0f;

  if (n > 0) {
    const u4_t* cp[RT];
    const uint16_t* sp[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      int64_t w = weight_row(a, row0 + rt * 16 + r16);
      if (w < 0) w = 0;  // read a valid row; the output is masked later
      cp[rt] = reinterpret_cast<const u4_t*>(a.packed + w * kh) + kq + 4 * (int64_t)g_begin;
      sp[rt] = a.scales + w * a.G + g_begin;
    }
    _Float16* xs = reinterpret_cast<_Float16*>(smem + wave * a.wave_lds);
    float accs[RT][4];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) accs[rt][r] = 0.0f;
    int E[TT];

    u4_t q[PD][RT];
    unsigned short sq[PD][RT];
#pragma unroll
    for (int s = 0; s < PD; ++s) {
      const int g = min(s, n - 1);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        q[s][rt] = __builtin_nontemporal_load(cp[rt] + 4 * g);
        sq[s][rt] = sp[rt][g];
      }
      __builtin_amdgcn_sched_barrier(0);  // issue in slot order, as the loop reloads them
    }

    for (int sb = 0; sb < n; sb += a.sk) {
      const int se = min(n, sb + a.sk);
      if (sb > 0) fold_slice<TT, RT>(acc, accs, E, kq);
      lds_fence();
      stage_wave<TT>(a, xs, g_begin + sb, g_begin + se, lane, E);
      // Staging already waited for its activation loads, issued after the
      // weight loads in flight; saying so lets the loop below wait for exactly
      // one group of weights at a time.
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      lds_fence();
      const _Float16* xr0 = xs + trow * a.xs_stride + kq * 32;
      for (int gi = sb; gi < se; gi += PD) {
#pragma unroll
        for (int s = 0; s < PD; ++s) {
          const int g = gi + s;
          const bool live = g < se;
          const _Float16* xr = xr0 + (min(g, se - 1) - sb) * kGroup;
          h8_t xa[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) xa[j] = *reinterpret_cast<const h8_t*>(xr + 8 * j);
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            const float sc = live ? bf16_to_f32(sq[s][rt]) : 0.0f;
            f4_t d = {0.0f, 0.0f, 0.0f, 0.0f};
            d = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[0], __builtin_bit_cast(h8_t, levels8(q[s][rt].x)), d, 0, 0, 0);
            d = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[1], __builtin_bit_cast(h8_t, levels8(q[s][rt].y)), d, 0, 0, 0);
            d = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[2], __builtin_bit_cast(h8_t, levels8(q[s][rt].z)), d, 0, 0, 0);
            d = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[3], __builtin_bit_cast(h8_t, levels8(q[s][rt].w)), d, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) accs[rt][r] = fmaf(d[r], sc, accs[rt][r]);
          }
          const int gn = min(g + PD, n - 1);
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            q[s][rt] = __builtin_nontemporal_load(cp[rt] + 4 * gn);
            sq[s][rt] = sp[rt][gn];
          }
          __builtin_amdgcn_sched_barrier(0);  // keep this slot's reloads here
        }
      }
    }
    fold_slice<TT, RT>(acc, accs, E, kq);
  }

  // Split-K partials of this wave -> its own LDS area: red[(rt*TT + t)*16 + row].
  lds_fence();
  float* red = reinterpret_cast<float*>(smem + wave * a.wave_lds);
  if (wave < a.nw) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = kq * 4 + r;
        if (t < TT) red[(rt * TT + t) * 16 + r16] = acc[rt][r];
      }
  }
  __syncthreads();

  float* fin = reinterpret_cast<float*>(smem + a.fin_offset);
  constexpr int kOut = RT * TT * 16;
  for (int o = threadIdx.x; o < kOut; o += blockDim.x) {
    float v = 0.0f;
    for (int w = 0; w < a.nw; ++w) v += reinterpret_cast<const float*>(smem + w * a.wave_lds)[o];
    const int rt = o / (TT * 16), t = (o >> 4) % TT, r = o & 15;
    const int64_t orow = row0 + rt * 16 + r;
    if (orow < a.n_out) {
      if (weight_row(a, orow) < 0) v = __builtin_nanf("");
      if (a.y) a.y[(int64_t)t * a.n_out + orow] = v;
    }
    fin[o] = v;
  }
  if (a.partial) {
    __syncthreads();
    if (wave == 0) workgroup_argmax<TT>(a, fin, row0, RT * 16, lane, wg);
  }
}

template <int TT, int RT, int PD>
__global__ void __launch_bounds__(512) w4a16_mfma_kernel(GemvArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  mfma_workgroup<TT, RT, PD>(a, blockIdx.x, smem);
}

// Grouped launch: workgroup b runs tile b - wg_start of the last problem whose
// wg_start <= b.
template <int TT, int RT, int PD>
__global__ void __launch_bounds__(512) w4a16_mfma_batch_kernel(const GemvArgs* __restrict__ table, int count) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int64_t b = blockIdx.x;
  int lo = 0, hi = count - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (table[mid].wg_start <= b)
      lo = mid;
    else
      hi = mid - 1;
  }
  const GemvArgs a = table[lo];
  mfma_workgroup<TT, RT, PD>(a, b - a.wg_start, smem);
}

// ----------------------------------------------------------------- dot ----

// Workgroup-cooperative staging of x[t][gs*128 .. ge*128) for the dot path.
template <int TT>
__device__ __forceinline__ void stage_block(const GemvArgs& a, _Float16* xs, unsigned* maxbuf, int gs, int ge,
                                            int (&E)[TT]) {
  const int n8 = (ge - gs) * (kGroup / 8);
  const int lane = threadIdx.x & 63, nw = blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    const u4_t* src = reinterpret_cast<const u4_t*>(a.x + (int64_t)t * a.K + (int64_t)gs * kGroup);
    unsigned m = 0;
    for (int b = threadIdx.x; b < n8; b += blockDim.x) m = max(m, absmax8(src[b]));
    m = wave_max(m);
    if (lane == 0) maxbuf[wave * TT + t] = m;
  }
  __syncthreads();
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    unsigned m = 0;
    for (int w = 0; w < nw; ++w) m = max(m, maxbuf[w * TT + t]);
    E[t] = slice_exponent(m);
    const u4_t* src = reinterpret_cast<const u4_t*>(a.x + (int64_t)t * a.K + (int64_t)gs * kGroup);
    u4_t* dst = reinterpret_cast<u4_t*>(xs + t * a.xs_stride);
    for (int b = threadIdx.x; b < n8; b += blockDim.x) dst[b] = convert8(src[b], E[t]);
  }
  __syncthreads();
}

// RW rows per wave, L = 64/RW lanes per row; a lane takes the row's 16-byte
// chunks li, li+L, li+2L, ...; CPL bounds the chunks per lane per slice.
template <int TT, int RW>
__global__ void __launch_bounds__(512) w4a16_dot_kernel(GemvArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  constexpr int L = 64 / RW;
  constexpr int CPL = 8;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;
  const int sub = lane / L, li = lane % L;
  const int64_t row0 = (int64_t)blockIdx.x * nw * RW;
  const int64_t orow = row0 + wave * RW + sub;
  int64_t w = weight_row(a, orow);
  const bool bad = w < 0;
  if (bad) w = 0;
  const u4_t* cp = reinterpret_cast<const u4_t*>(a.packed + w * (int64_t)(a.K >> 1));
  const uint16_t* sp = a.scales + w * a.G;
  _Float16* xs = reinterpret_cast<_Float16*>(smem);
  unsigned* maxbuf = reinterpret_cast<unsigned*>(smem + a.fin_offset);

  float acc[TT], accs[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) acc[t] = accs[t] = 0.0f;
  int E[TT];

  for (int gs = 0; gs < a.G; gs += a.sk) {
    const int ge = min(a.G, gs + a.sk);
    const int c0 = gs * 4, nc = (ge - gs) * 4;  // 16-byte chunks of this slice
    u4_t q[CPL];
    unsigned short sq[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = li + i * L;
      if (c < nc) {
        q[i] = __builtin_nontemporal_load(cp + c0 + c);
        sq[i] = sp[(c0 + c) >> 2];
      }
    }
    if (gs > 0) __syncthreads();  // every wave is done with the previous slice
    stage_block<TT>(a, xs, maxbuf, gs, ge, E);
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = li + i * L;
      if (c < nc) {
        const u4_t lv[4] = {levels8(q[i].x), levels8(q[i].y), levels8(q[i].z), levels8(q[i].w)};
        const float sc = bf16_to_f32(sq[i]);
#pragma unroll
        for (int t = 0; t < TT; ++t) {
          const u4_t* xv = reinterpret_cast<const u4_t*>(xs + t * a.xs_stride + c * 32);
          float p = 0.0f;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const u4_t xw = xv[j];
            p = dot2(lv[j].x, xw.x, p);
            p = dot2(lv[j].y, xw.y, p);
            p = dot2(lv[j].z, xw.z, p);
            p = dot2(lv[j].w, xw.w, p);
          }
          accs[t] = fmaf(p, sc, accs[t]);
        }
      }
    }
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      acc[t] += ldexpf(accs[t], -E[t]);
      accs[t] = 0.0f;
    }
  }

  // Butterfly across the L lanes of a row (fixed order).
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int off = L / 2; off >= 1; off >>= 1) acc[t] += __shfl_xor(acc[t], off);

  float* fin = reinterpret_cast<float*>(smem);  // reused after the last slice
  __syncthreads();
  if (li == 0) {
    const int r = wave * RW + sub;  // row within the workgroup
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      float v = bad ? __builtin_nanf("") : acc[t];
      if (orow < a.n_out && a.y) a.y[(int64_t)t * a.n_out + orow] = v;
      fin[((r >> 4) * TT + t) * 16 + (r & 15)] = v;
    }
  }
  if (a.partial) {
    __syncthreads();
    if (wave == 0) workgroup_argmax<TT>(a, fin, row0, nw * RW, lane, blockIdx.x);
  }
}

// -------------------------------------------------------------- stream ----

// Weight-code load of the streaming kernel.  Default cache policy: the two
// 64-byte halves of a 128-byte line (groups g and g+1 of a row) then merge
// into one L2 request in the vector L1; the nontemporal hint would send each
// half on its own and double the requests in flight.
__device__ __forceinline__ u4_t load_codes(const u4_t* p) { return *p; }

// bf16 scale e of eight packed in v (element order = memory order) -> fp32.
__device__ __forceinline__ float scale_of(u4_t v, int e) {
  const unsigned w = (e >> 1) == 0 ? v.x : (e >> 1) == 1 ? v.y : (e >> 1) == 2 ? v.z : v.w;
  return __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
}

// The K loop of one wave of the streaming kernel: PD groups of codes in
// flight.  VS: the row's scales are read eight groups (16 bytes) at a time,
// one load per 8 groups instead of one per group (needs G % 8 == 0 and
// 16-byte aligned scale rows); otherwise one 2-byte load per group.
template <int TT, int PD, bool VS>
__device__ __forceinline__ void stream_rows(const GemvArgs& a, const u4_t* cp, const uint16_t* sp, _Float16* xs,
                                            unsigned* maxbuf, int trow, int kq, float (&acc)[1][4]) {
  constexpr int NV = VS ? PD / 8 : 1;  // scale vectors per ring cycle
  static_assert(!VS || PD % 8 == 0, "vector scales need PD % 8 == 0");
  const int G = a.G;
  float accs[1][4];
#pragma unroll
  for (int r = 0; r < 4; ++r) accs[0][r] = 0.0f;
  int E[TT];

  // The first slice is staged before any weight load is issued.
  int se = min(G, a.sk);
  stage_block<TT>(a, xs, maxbuf, 0, se, E);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

  const u4_t* svp = reinterpret_cast<const u4_t*>(sp);
  const int nvec = G / 8;
  u4_t sv[NV];
  if constexpr (VS) {
#pragma unroll
    for (int c = 0; c < NV; ++c) sv[c] = svp[min(c, nvec - 1)];
  }
  u4_t q[PD];
  unsigned short sq[PD];
#pragma unroll
  for (int s = 0; s < PD; ++s) {
    const int g = min(s, G - 1);
    if constexpr (!VS) sq[s] = sp[g];
    q[s] = load_codes(cp + 4 * g);
    __builtin_amdgcn_sched_barrier(0);  // issue in slot order, as the loop reloads them
  }
  for (int sb = 0; sb < G; sb += a.sk) {
    se = min(G, sb + a.sk);
    if (sb > 0) {
      fold_slice<TT, 1>(acc, accs, E, kq);
      __syncthreads();  // every wave is done with the previous slice
      stage_block<TT>(a, xs, maxbuf, sb, se, E);
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    }
    const _Float16* xr0 = xs + trow * a.xs_stride + kq * 32;
    for (int gi = sb; gi < se; gi += PD) {
      u4_t svn[NV];
      if constexpr (VS) {
#pragma unroll
        for (int c = 0; c < NV; ++c) svn[c] = svp[min(gi / 8 + NV + c, nvec - 1)];
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int s = 0; s < PD; ++s) {
        const int g = gi + s;
        const _Float16* xr = xr0 + (min(g, se - 1) - sb) * kGroup;
        h8_t xa[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) xa[j] = *reinterpret_cast<const h8_t*>(xr + 8 * j);
        float sc;
        if constexpr (VS)
          sc = scale_of(sv[s / 8], s % 8);
        else
          sc = bf16_to_f32(sq[s]);
        sc = (g < se) ? sc : 0.0f;
        f4_t d = {0.0f, 0.0f, 0.0f, 0.0f};
        d = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[0], __builtin_bit_cast(h8_t, levels8(q[s].x)), d, 0, 0, 0);
        d = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[1], __builtin_bit_cast(h8_t, levels8(q[s].y)), d, 0, 0, 0);
        d = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[2], __builtin_bit_cast(h8_t, levels8(q[s].z)), d, 0, 0, 0);
        d = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[3], __builtin_bit_cast(h8_t, levels8(q[s].w)), d, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) accs[0][r] = fmaf(d[r], sc, accs[0][r]);
        const int gn = min(g + PD, G - 1);
        if constexpr (!VS) sq[s] = sp[gn];
        q[s] = load_codes(cp + 4 * gn);
        // keep this slot's reload here: sunk to the end of the loop, the
        // reloads would make every iteration wait for the whole ring
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (VS) {
#pragma unroll
        for (int c = 0; c < NV; ++c) sv[c] = svn[c];
      }
    }
  }
  fold_slice<TT, 1>(acc, accs, E, kq);
}

// Streaming variant of the matrix-core path: each wave owns one 16-row tile
// over all of K and keeps PD groups of its rows in flight (PD x 64 bytes of
// every row requested together, which is what lets the 16-row x 64-byte
// access pattern of the MFMA operand layout stream at full HBM rate); the
// waves of a workgroup share one staged copy of the activations per K slice,
// so the fp16 conversion is paid once per 16 * (waves) rows.  No split-K:
// every output comes straight from one wave's registers.
template <int TT, int PD>
__device__ __forceinline__ void stream_workgroup(const GemvArgs& a, int64_t wg, unsigned char* smem) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nwv = blockDim.x >> 6;
  const int r16 = lane & 15, kq = lane >> 4;
  const int trow = min(r16, TT - 1);
  const int64_t tile0 = (wg * nwv + wave) * 16;
  const int64_t kh = a.K >> 1;
  int64_t w = weight_row(a, tile0 + r16);
  if (w < 0) w = 0;
  const u4_t* cp = reinterpret_cast<const u4_t*>(a.packed + w * kh) + kq;
  const uint16_t* sp = a.scales + w * a.G;
  _Float16* xs = reinterpret_cast<_Float16*>(smem);
  unsigned* maxbuf = reinterpret_cast<unsigned*>(smem + a.fin_offset);

  float acc[1][4];
#pragma unroll
  for (int r = 0; r < 4; ++r) acc[0][r] = 0.0f;
  if (a.vec_scales)
    stream_rows<TT, PD, true>(a, cp, sp, xs, maxbuf, trow, kq, acc);
  else
    stream_rows<TT, PD, false>(a, cp, sp, xs, maxbuf, trow, kq, acc);

  const int64_t orow = tile0 + r16;
  const bool in_range = orow < a.n_out;
  const bool bad = in_range && weight_row(a, orow) < 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = kq * 4 + r;
    if (t < TT && in_range && a.y) a.y[(int64_t)t * a.n_out + orow] = bad ? __builtin_nanf("") : acc[0][r];
  }
  if (a.partial) {
    // per t: best (value, id) of this wave's 16 rows, then of the workgroup
    int2* fin = reinterpret_cast<int2*>(smem + a.fin_offset);
    __syncthreads();  // staging area and max buffer are free now
    const int64_t vid = (in_range && !bad) ? (a.row_ids ? (int64_t)a.row_ids[orow] : orow) : -1;
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      const int r = t & 3;
      float v = acc[0][0];
#pragma unroll
      for (int i = 1; i < 4; ++i) v = (r == i) ? acc[0][i] : v;
      int id = (kq == (t >> 2) && vid >= 0 && !__builtin_isnan(v)) ? (int)vid : -1;
      if (id < 0) v = __builtin_nanf("");
      wave_argmax(v, id);
      if (lane == 0) fin[wave * TT + t] = int2{__float_as_int(v), id};
    }
    __syncthreads();
    if (wave == 0 && lane < TT) {
      float bv = __builtin_nanf("");
      int bi = -1;
      for (int w2 = 0; w2 < nwv; ++w2) {
        const int2 c = fin[w2 * TT + lane];
        if (better(__int_as_float(c.x), c.y, bv, bi)) {
          bv = __int_as_float(c.x);
          bi = c.y;
        }
      }
      a.partial[wg * TT + lane] = int2{__float_as_int(bv), bi};
    }
  }
}

template <int TT, int PD>
__global__ void __launch_bounds__(256) w4a16_stream_kernel(GemvArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  stream_workgroup<TT, PD>(a, blockIdx.x, smem);
}

template <int TT, int PD>
__global__ void __launch_bounds__(256) w4a16_stream_batch_kernel(const GemvArgs* __restrict__ table, int count) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int64_t b = blockIdx.x;
  int lo = 0, hi = count - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (table[mid].wg_start <= b)
      lo = mid;
    else
      hi = mid - 1;
  }
  const GemvArgs a = table[lo];
  stream_workgroup<TT, PD>(a, b - a.wg_start, smem);
}

// ---------------------------------------------------------- argmax final ----

__global__ void __launch_bounds__(256) w4a16_argmax_final(const int2* partial, int64_t nparts, int T, int32_t* id_out,
                                                          float* val_out) {
  __shared__ float sv[4];
  __shared__ int si[4];
  const int t = blockIdx.x;
  float bv = __builtin_nanf("");
  int bi = -1;
  for (int64_t j = threadIdx.x; j < nparts; j += blockDim.x) {
    const int2 p = partial[j * T + t];
    const float v = __int_as_float(p.x);
    if (better(v, p.y, bv, bi)) {
      bv = v;
      bi = p.y;
    }
  }
  wave_argmax(bv, bi);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    sv[wave] = bv;
    si[wave] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < (int)(blockDim.x >> 6); ++w)
      if (better(sv[w], si[w], bv, bi)) {
        bv = sv[w];
        bi = si[w];
      }
    if (id_out) id_out[t] = bi;
    if (val_out) val_out[t] = bi < 0 ? __builtin_nanf("") : bv;
  }
}

// ------------------------------------------------------------- dispatch ----

// (RT, PD) pairs the mfma kernels are built for.
#define W4A16_MFMA_SHAPES(X) X(1, 2) X(1, 4) X(1, 8) X(4, 2) X(4, 4)

template <int TT>
hipError_t launch_t(const GemvArgs& a, const GemvArgs* table, int count, const Plan& p, hipStream_t s) {
  const dim3 grid((unsigned)p.grid), block((unsigned)p.threads);
  if (p.variant == 2) {
#define W4A16_CASE(R, D)                                                                                \
  if (p.rt == R && p.pd == D) {                                                                         \
    if (table)                                                                                          \
      hipLaunchKernelGGL((w4a16_mfma_batch_kernel<TT, R, D>), grid, block, p.lds, s, table, count);     \
    else                                                                                                \
      hipLaunchKernelGGL((w4a16_mfma_kernel<TT, R, D>), grid, block, p.lds, s, a);                      \
    return hipGetLastError();                                                                           \
  }
    W4A16_MFMA_SHAPES(W4A16_CASE)
#undef W4A16_CASE
    return hipErrorInvalidValue;
  }
  if (p.variant == 3) {
#define W4A16_CASE(D)                                                                                   \
  if (p.pd == D) {                                                                                      \
    if (table)                                                                                          \
      hipLaunchKernelGGL((w4a16_stream_batch_kernel<TT, D>), grid, block, p.lds, s, table, count);      \
    else                                                                                                \
      hipLaunchKernelGGL((w4a16_stream_kernel<TT, D>), grid, block, p.lds, s, a);                       \
    return hipGetLastError();                                                                           \
  }
    W4A16_CASE(8)
    W4A16_CASE(16)
#undef W4A16_CASE
    return hipErrorInvalidValue;
  }
  if (table || p.rt != 2) return hipErrorInvalidValue;
  hipLaunchKernelGGL((w4a16_dot_kernel<TT, 2>), grid, block, p.lds, s, a);
  return hipGetLastError();
}

template <typename F>
hipError_t for_t(int T, F&& f) {
  switch (T) {
    case 1: return f(std::integral_constant<int, 1>{});
    case 2: return f(std::integral_constant<int, 2>{});
    case 3: return f(std::integral_constant<int, 3>{});
    case 4: return f(std::integral_constant<int, 4>{});
    case 5: return f(std::integral_constant<int, 5>{});
    case 6: return f(std::integral_constant<int, 6>{});
    case 7: return f(std::integral_constant<int, 7>{});
    case 8: return f(std::integral_constant<int, 8>{});
    default: return hipErrorInvalidValue;
  }
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// W4A16_STREAM="pd,waves" overrides the streaming tile (for measurement).
void stream_override(int* pd, int* nwv) {
  if (const char* e = std::getenv("W4A16_STREAM")) {
    int x = 0, y = 0;
    if (std::sscanf(e, "%d,%d", &x, &y) == 2 && (x == 8 || x == 16) && y >= 1 && y <= 4) {
      *pd = x;
      *nwv = y;
    }
  }
}

}  // namespace

// Tiling of one problem for a fixed tile height (rt), prefetch depth (pd)
// and at most nw_max waves.  K is split into per-wave ranges of gpw groups, a
// multiple of pd (the last wave may hold fewer); the activation slice staged
// in LDS holds sk groups (all of a wave's range when 64 KB allow it, else a
// multiple of pd).
void plan_mfma_fixed(GemvArgs& a, int T, int rt, int pd, int nw_max, int* lds, int64_t* grid) {
  const int fin_bytes = rt * T * 16 * 4;
  int nw = std::max(1, std::min(nw_max, a.G));
  int gpw = 0, nw_eff = 0, sk = 0;
  for (;; --nw) {
    gpw = (int)(cdiv(cdiv(a.G, nw), pd) * pd);
    nw_eff = (int)cdiv(a.G, gpw);
    const int per_wave = (kLdsCap - fin_bytes) / nw_eff;
    sk = (per_wave / T - 16) / (kGroup * 2);
    if (sk >= gpw) {
      sk = gpw;
      break;
    }
    if (sk >= pd || nw == 1) {
      sk = std::max(pd, sk - sk % pd);
      break;
    }
  }
  a.nw = nw_eff;
  a.gpw = gpw;
  a.sk = sk;
  a.xs_stride = sk * kGroup + 8;  // 16-byte pad between token rows
  int wave_lds = std::max(T * a.xs_stride * 2, rt * T * 16 * 4);
  a.wave_lds = (wave_lds + 15) & ~15;
  a.fin_offset = nw_eff * a.wave_lds;
  *lds = a.fin_offset + fin_bytes;
  *grid = cdiv(cdiv(a.n_out, 16), rt);
}

// Tiling of a single matrix-core launch.  Tall matrices (>= 1024 tiles of
// 16 rows) stream: one wave per 16-row tile over all of K, four waves per
// workgroup sharing the staged activations.  Shorter ones split K over the
// waves of a workgroup (16 rows per workgroup) so that they still put ~12
// waves of weight loads on every CU; the prefetch depth is the largest the
// per-wave K range fills.
Plan plan_mfma(GemvArgs& a, int T) {
  Plan p{};
  const int64_t tiles = cdiv(a.n_out, 16);
  if (tiles >= 1024) {
    p.variant = 3;
    p.rt = 1;
    p.pd = (a.G % 16 == 0) ? 16 : 8;
    int nwv = 4;
    stream_override(&p.pd, &nwv);
    plan_stream(a, T, p.pd, nwv, &p.lds, &p.grid);
    p.threads = nwv * 64;
    return p;
  }
  p.variant = 2;
  p.rt = 1;
  const int nw_max = (int)std::min<int64_t>(8, std::max<int64_t>(1, cdiv(3072, tiles)));
  const int gpw_est = (int)cdiv(a.G, std::min(nw_max, a.G));
  p.pd = gpw_est >= 8 ? 8 : (gpw_est >= 4 ? 4 : 2);
  plan_mfma_fixed(a, T, p.rt, p.pd, nw_max, &p.lds, &p.grid);
  p.threads = a.nw * 64;
  return p;
}

// Tiling of the streaming variant: nwv waves (16-row tiles) per workgroup,
// the activation slice staged in LDS holds sk groups (all of K when 64 KB
// allow it, else a multiple of pd).
void plan_stream(GemvArgs& a, int T, int pd, int nwv, int* lds, int64_t* grid) {
  a.vec_scales = (a.G % 8 == 0 && (reinterpret_cast<uintptr_t>(a.scales) & 15) == 0) ? 1 : 0;
  const int small = std::max(nwv * T * 4, nwv * T * 8);  // max buffer / argmax partials
  int sk = ((kLdsCap - small - 16) / T - 16) / (kGroup * 2);
  if (sk < a.G) sk = std::max(pd, sk - sk % pd);
  else sk = a.G;
  a.nw = nwv;
  a.gpw = a.G;
  a.sk = sk;
  a.xs_stride = sk * kGroup + 8;
  a.wave_lds = 0;
  a.fin_offset = (T * a.xs_stride * 2 + 15) & ~15;
  *lds = a.fin_offset + small;
  *grid = cdiv(a.n_out, 16LL * nwv);
}

// Tiling of the dot variant: 2 rows per wave (32 lanes per row), 8 waves,
// activations staged per workgroup in slices of at most 8 chunks per lane.
Plan plan_dot(GemvArgs& a, int T) {
  Plan p{};
  p.variant = 1;
  p.rt = 2;  // rows per wave
  const int nw = 8;
  p.threads = nw * 64;
  const int L = 64 / p.rt;
  p.grid = cdiv(a.n_out, (int64_t)p.rt * nw);
  const int max_sk_regs = 8 * L / 4;  // CPL chunks per lane, 4 chunks per group
  const int fin_bytes = std::max(nw * T * 4, (int)cdiv(nw * p.rt, 16) * T * 16 * 4);
  int sk_lds = ((kLdsCap - fin_bytes) / T - 16) / (kGroup * 2);
  a.nw = nw;
  a.sk = std::max(1, std::min({a.G, max_sk_regs, sk_lds}));
  a.gpw = a.G;
  a.xs_stride = a.sk * kGroup + 8;
  a.wave_lds = 0;
  int xs_bytes = T * a.xs_stride * 2;
  xs_bytes = std::max(xs_bytes, (int)cdiv(nw * p.rt, 16) * T * 16 * 4);  // also holds final values
  a.fin_offset = (xs_bytes + 15) & ~15;                                 // max buffer follows
  p.lds = a.fin_offset + nw * T * 4;
  return p;
}

int64_t max_workgroups(int64_t n_out) { return cdiv(n_out, 16); }

hipError_t launch(const GemvArgs& a, const Plan& p, int T, hipStream_t s) {
  return for_t(T, [&](auto tt) { return launch_t<decltype(tt)::value>(a, nullptr, 0, p, s); });
}

hipError_t launch_batch(const GemvArgs* table_dev, int count, const Plan& p, int T, hipStream_t s) {
  GemvArgs unused{};
  return for_t(T, [&](auto tt) { return launch_t<decltype(tt)::value>(unused, table_dev, count, p, s); });
}

hipError_t launch_argmax_final(const int2* partial, int64_t nparts, int T, int32_t* id, float* val, hipStream_t s) {
  hipLaunchKernelGGL(w4a16_argmax_final, dim3((unsigned)T), dim3(256), 0, s, partial, nparts, T, id, val);
  return hipGetLastError();
}

}  // namespace w4a16
