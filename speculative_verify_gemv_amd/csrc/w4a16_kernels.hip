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

__device__ __forceinline__ float bf16_to_f32(unsigned short b) { return __uint_as_float((unsigned)b << 16); }

template <typename V>
__device__ __forceinline__ unsigned as_u32(V h) {
  static_assert(sizeof(V) == 4, "packed pair");
  return __builtin_bit_cast(unsigned, h);
}

// Eight exact fp16 levels (q - 8) of one word, slot order 0,4,1,5,2,6,3,7.
__device__ __forceinline__ u4_t levels8(unsigned w) {
  const unsigned w8 = w >> 8;
  const h2_t lo_bias = {(_Float16)-1032.0f, (_Float16)-1032.0f};
  const h2_t hi_bias = {(_Float16)-72.0f, (_Float16)-72.0f};
  const h2_t a = __builtin_bit_cast(h2_t, (w & 0x000F000Fu) | 0x64006400u) + lo_bias;
  const h2_t b = __builtin_bit_cast(h2_t, (w & 0x00F000F0u) | 0x54005400u) + hi_bias;
  const h2_t c = __builtin_bit_cast(h2_t, (w8 & 0x000F000Fu) | 0x64006400u) + lo_bias;
  const h2_t d = __builtin_bit_cast(h2_t, (w8 & 0x00F000F0u) | 0x54005400u) + hi_bias;
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
                                                 int lane) {
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
    if (lane == 0) a.partial[(int64_t)blockIdx.x * TT + t] = int2{__float_as_int(bv), bi};
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

template <int TT, int RT>
__global__ void __launch_bounds__(512) w4a16_mfma_kernel(GemvArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  constexpr int PD = (RT == 1) ? 4 : 2;  // groups of weight loads kept in flight per wave
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const int r16 = lane & 15;  // output row of the B operand / token row of the A operand
  const int kq = lane >> 4;   // quarter of the 128-column group
  const int64_t row0 = (int64_t)blockIdx.x * (RT * 16);
  const int64_t kh = a.K >> 1;

  const u4_t* cp[RT];
  const uint16_t* sp[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    int64_t w = weight_row(a, row0 + rt * 16 + r16);
    if (w < 0) w = 0;  // read a valid row; the output is masked below
    cp[rt] = reinterpret_cast<const u4_t*>(a.packed + w * kh) + kq;
    sp[rt] = a.scales + w * a.G;
  }

  const int g_begin = wave * a.gpw;
  const int g_end = min(a.G, g_begin + a.gpw);
  _Float16* xs = reinterpret_cast<_Float16*>(smem + wave * a.wave_lds);

  float acc[RT][4], accs[RT][4];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[rt][r] = accs[rt][r] = 0.0f;
  int E[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) E[t] = 0;

  u4_t q[PD][RT];
  unsigned short sq[PD][RT];
#pragma unroll
  for (int s = 0; s < PD; ++s)
    if (g_begin + s < g_end)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        q[s][rt] = __builtin_nontemporal_load(cp[rt] + 4 * (g_begin + s));
        sq[s][rt] = sp[rt][g_begin + s];
      }

  int slice_begin = g_begin, slice_end = g_begin;
  for (int gb = g_begin; gb < g_end; gb += PD) {
    if (gb >= slice_end) {
      if (gb > g_begin) fold_slice<TT, RT>(acc, accs, E, kq);
      lds_fence();
      slice_begin = gb;
      slice_end = min(g_end, gb + a.sk);
      stage_wave<TT>(a, xs, slice_begin, slice_end, lane, E);
      lds_fence();
    }
#pragma unroll
    for (int s = 0; s < PD; ++s) {
      const int g = gb + s;
      if (g < g_end) {
        h8_t xa[4];
        const _Float16* xr = xs + r16 * a.xs_stride + (g - slice_begin) * kGroup + kq * 32;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (r16 < TT)
            xa[j] = *reinterpret_cast<const h8_t*>(xr + 8 * j);
          else
            xa[j] = h8_t{};
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const float sc = bf16_to_f32(sq[s][rt]);
          f4_t d = {0.0f, 0.0f, 0.0f, 0.0f};
          d = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[0], __builtin_bit_cast(h8_t, levels8(q[s][rt].x)), d, 0, 0, 0);
          d = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[1], __builtin_bit_cast(h8_t, levels8(q[s][rt].y)), d, 0, 0, 0);
          d = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[2], __builtin_bit_cast(h8_t, levels8(q[s][rt].z)), d, 0, 0, 0);
          d = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[3], __builtin_bit_cast(h8_t, levels8(q[s][rt].w)), d, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r) accs[rt][r] = fmaf(d[r], sc, accs[rt][r]);
        }
        if (g + PD < g_end)
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            q[s][rt] = __builtin_nontemporal_load(cp[rt] + 4 * (g + PD));
            sq[s][rt] = sp[rt][g + PD];
          }
      }
    }
  }
  if (g_end > g_begin) fold_slice<TT, RT>(acc, accs, E, kq);

  // Split-K partials of this wave -> its own LDS area: red[(rt*TT + t)*16 + row].
  lds_fence();
  float* red = reinterpret_cast<float*>(smem + wave * a.wave_lds);
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = kq * 4 + r;
      if (t < TT) red[(rt * TT + t) * 16 + r16] = acc[rt][r];
    }
  __syncthreads();

  float* fin = reinterpret_cast<float*>(smem + a.fin_offset);
  constexpr int kOut = RT * TT * 16;
  for (int o = threadIdx.x; o < kOut; o += blockDim.x) {
    float v = 0.0f;
    for (int w = 0; w < nw; ++w) v += reinterpret_cast<const float*>(smem + w * a.wave_lds)[o];
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
    if (wave == 0) workgroup_argmax<TT>(a, fin, row0, RT * 16, lane);
  }
}

// ----------------------------------------------------------------- dot ----

// Workgroup-cooperative staging of x[t][gs*128 .. ge*128) for the dot path.
template <int TT>
__device__ __forceinline__ void stage_block(const GemvArgs& a, _Float16* xs, unsigned* maxbuf, int gs, int ge,
                                            int (&E)[TT]) {
  const int n8 = (ge - gs) * (kGroup / 8);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
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
  const int wave = threadIdx.x >> 6;
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
    if (wave == 0) workgroup_argmax<TT>(a, fin, row0, nw * RW, lane);
  }
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

template <int TT>
hipError_t launch_t(const GemvArgs& a, const Plan& p, hipStream_t s) {
  const dim3 grid((unsigned)p.grid), block((unsigned)(p.nw * 64));
  if (p.variant == 2) {
    switch (p.rt) {
      case 1: hipLaunchKernelGGL((w4a16_mfma_kernel<TT, 1>), grid, block, p.lds, s, a); break;
      case 2: hipLaunchKernelGGL((w4a16_mfma_kernel<TT, 2>), grid, block, p.lds, s, a); break;
      case 4: hipLaunchKernelGGL((w4a16_mfma_kernel<TT, 4>), grid, block, p.lds, s, a); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (p.rt) {
      case 1: hipLaunchKernelGGL((w4a16_dot_kernel<TT, 1>), grid, block, p.lds, s, a); break;
      case 2: hipLaunchKernelGGL((w4a16_dot_kernel<TT, 2>), grid, block, p.lds, s, a); break;
      case 4: hipLaunchKernelGGL((w4a16_dot_kernel<TT, 4>), grid, block, p.lds, s, a); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

// Tiling of the mfma variant.  Enough workgroups to cover the 256 CUs
// (16-row tiles, grouped by 2 or 4 for large heads so activations are staged
// once per 32 or 64 rows); the waves of a workgroup split K so that a small
// matrix still puts ~12 waves of weight loads on every CU.
Plan plan_mfma(GemvArgs& a, int T) {
  Plan p{};
  p.variant = 2;
  const int64_t tiles = cdiv(a.n_out, 16);
  p.rt = tiles >= 2048 ? 4 : (tiles >= 768 ? 2 : 1);
  p.grid = cdiv(tiles, p.rt);
  const int pd = (p.rt == 1) ? 4 : 2;  // prefetch depth of the kernel; slices are multiples of it
  const int fin_bytes = p.rt * T * 16 * 4;
  int nw = (int)std::min<int64_t>(8, std::max<int64_t>(1, cdiv(3072, p.grid)));
  nw = std::min(nw, a.G);
  int gpw = 0, sk = 0;
  for (;; --nw) {
    gpw = (int)cdiv(a.G, nw);
    const int nw_eff = (int)cdiv(a.G, gpw);
    const int per_wave = (kLdsCap - fin_bytes) / nw_eff;
    sk = (per_wave / T - 16) / (kGroup * 2);
    if (sk >= gpw) {
      sk = gpw;
      nw = nw_eff;
      break;
    }
    if (sk >= pd || nw == 1) {
      sk = std::max(pd, sk - sk % pd);
      nw = nw_eff;
      break;
    }
  }
  p.nw = nw;
  a.gpw = gpw;
  a.sk = sk;
  a.xs_stride = sk * kGroup + 8;  // 16-byte pad between token rows
  int wave_lds = T * a.xs_stride * 2;
  wave_lds = std::max(wave_lds, p.rt * T * 16 * 4);
  a.wave_lds = (wave_lds + 15) & ~15;
  a.fin_offset = nw * a.wave_lds;
  p.lds = a.fin_offset + fin_bytes;
  return p;
}

// Tiling of the dot variant: 2 rows per wave (32 lanes per row), 8 waves,
// activations staged per workgroup in slices of at most 8 chunks per lane.
Plan plan_dot(GemvArgs& a, int T) {
  Plan p{};
  p.variant = 1;
  p.rt = 2;  // rows per wave
  p.nw = 8;
  const int L = 64 / p.rt;
  p.grid = cdiv(a.n_out, (int64_t)p.rt * p.nw);
  const int max_sk_regs = 8 * L / 4;  // CPL chunks per lane, 4 chunks per group
  const int fin_bytes = std::max(p.nw * T * 4, (int)cdiv(p.nw * p.rt, 16) * T * 16 * 4);
  int sk_lds = ((kLdsCap - fin_bytes) / T - 16) / (kGroup * 2);
  a.sk = std::max(1, std::min({a.G, max_sk_regs, sk_lds}));
  a.gpw = a.G;
  a.xs_stride = a.sk * kGroup + 8;
  a.wave_lds = 0;
  int xs_bytes = T * a.xs_stride * 2;
  xs_bytes = std::max(xs_bytes, (int)cdiv(p.nw * p.rt, 16) * T * 16 * 4);  // also holds final values
  a.fin_offset = (xs_bytes + 15) & ~15;                                  // max buffer follows
  p.lds = a.fin_offset + p.nw * T * 4;
  return p;
}

int64_t max_workgroups(int64_t n_out) { return cdiv(n_out, 16); }

hipError_t launch(const GemvArgs& a, const Plan& p, int T, hipStream_t s) {
  switch (T) {
    case 1: return launch_t<1>(a, p, s);
    case 2: return launch_t<2>(a, p, s);
    case 3: return launch_t<3>(a, p, s);
    case 4: return launch_t<4>(a, p, s);
    case 5: return launch_t<5>(a, p, s);
    case 6: return launch_t<6>(a, p, s);
    case 7: return launch_t<7>(a, p, s);
    case 8: return launch_t<8>(a, p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_argmax_final(const int2* partial, int64_t nparts, int T, int32_t* id, float* val, hipStream_t s) {
  hipLaunchKernelGGL(w4a16_argmax_final, dim3((unsigned)T), dim3(256), 0, s, partial, nparts, T, id, val);
  return hipGetLastError();
}

}  // namespace w4a16
