// Device code of libw4a16 for gfx950 (CDNA4), shared by the translation
// units that instantiate it: w4a16_kernels_tt.hip builds launch_t<TT> for
// one activation-row count TT per object, so the kernels compile in
// parallel; w4a16_kernels.hip holds the planning, the dispatch and the
// non-template kernels.
//
// W4A16 skinny matmul kernels for AMD Instinct MI355X (gfx950, CDNA4).
//
// y[t][n] = sum_k (q[n][k] - 8) * scale[n][k/128] * x[t][k]   (fp32 out)
//
// The weight format -- little-endian words of eight nibbles, level = nibble
// minus 8, one bf16 scale per 128 columns applied after the group's sum -- is
// the one the qwen-warp/llamAmpere article gives under "qwen-warp: keep the
// activations in bf16".  As in that engine, the activations stay bf16 and
// the matrix cores multiply them with bf16 levels, so every product
// (q - 8) * x is exact in fp32 for every finite bf16 x: the activations are
// copied into LDS as they are, with no conversion and no range rule.  That
// engine makes a bf16 level pair with one OR and one packed bf16 FMA; gfx950
// has no packed bf16 arithmetic, so here a word w of eight codes becomes
// eight exact levels like this:
//
//   e = w ^ 0x88888888   every nibble becomes the 4-bit two's complement of
//                        q - 8 (q ^ 8 read as a signed nibble)
//   v_cvt_off_f32_i4     a signed nibble n (bits 0-3 of a byte picked by an
//                        SDWA byte select, of e and of e >> 4) -> n / 16 as an
//                        fp32, exact
//   v_perm_b32           the high halves of two such floats -> one bf16 pair
//                        (a float with at most 4 significant bits equals its
//                        own top 16 bits read as a bf16)
//
// 14 VALU operations per word, levels in natural k order.  The levels carry
// a factor 1/16, which is taken back when a tile's sum is folded (a power of
// two), so the result is the fp32 arithmetic of the unscaled levels.
//
// Where the loop is tight those 14 operations cost about 4.5% of the
// bandwidth, so the kernels first try a cheaper exact form (all row counts
// where a workgroup stages the activations for its waves, up to two rows
// where each wave stages its own): fp16 levels, 9 operations per word,
//
//   (w & 0x000F000F) | 0x6400_6400  is the fp16 pair (1024 + q0, 1024 + q4)
//   (w & 0x00F000F0) | 0x5400_5400  is the fp16 pair (  64 + q1,   64 + q5)
//
// (at 1024 the fp16 spacing is 1, at 64 it is 1/16 and the nibble sits four
// bits higher), then one v_pk_add_f16 with -1032 / -72 each, against
// activations converted to fp16 times a power of two 2^E.  That conversion
// is exact when every scaled magnitude lies in [2^-17, 65280] (or is zero):
// a staged slice tries E = kDirectE (magnitudes in [2^-21, 4080]), then the
// E its own range allows; a slice that no E fits is staged as the bf16
// values they are and runs the bf16 levels.  Both forms give exact products
// and fp32 sums, so the choice changes rounding order at most, never the
// tolerance.
//
// Two variants:
//  * matrix core: tokens are the A operand of v_mfma_f32_16x16x32_bf16 (T
//    padded to 16 rows), weights the B operand (16 output rows x 32 k).  A
//    lane owns one output row and a quarter of each 128-column group, loads
//    its 16 bytes of that group with one 128-bit load, and feeds the four
//    words to four MFMAs.  Each 128-column group gets a fresh accumulator
//    that is then scaled in fp32.  A wave streams RT 16-row tiles one after
//    the other with eight groups of loads in flight.  In a "shared"
//    workgroup the waves own different tiles and share one staged copy of
//    the activations; in a "split" workgroup they split K over the same
//    tiles and add their partial sums through LDS in wave order.
//  * dot: lanes split a row's K in 16-byte chunks; v_dot2_f32_bf16 forms each
//    chunk's partial, which is scaled by its group scale; the 32 lanes of a
//    row are reduced with DPP row operations and one ds_swizzle.
//
// Both reduce in an order fixed by (K, tiling) only, so results are
// deterministic, and identical weight rows give identical outputs.
#pragma once
#include <math.h>

#include <algorithm>
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <type_traits>

#include "w4a16_internal.h"

namespace w4a16 {
namespace {

typedef __bf16 b8_t __attribute__((ext_vector_type(8)));  // the bf16 MFMA builtin's operand type
typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
typedef __fp16 h8_t __attribute__((ext_vector_type(8)));  // the fp16 MFMA builtin's operand type
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef unsigned short us2_t __attribute__((ext_vector_type(2)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef unsigned u4_t __attribute__((ext_vector_type(4)));

constexpr int kGroup = 128;
constexpr int kLdsCap = 65536;  // dynamic LDS per workgroup (several workgroups per CU)
constexpr int kCuLds = 163840;  // LDS of a CU (one workgroup per CU)
constexpr int kRing = 8;        // groups of weight codes in flight per wave
// s_waitcnt immediate (gfx9 encoding) waiting for vmcnt = 0 only.
constexpr int kWaitVmcnt0 = 0x0F70;
// The bf16 levels are (q - 8) / 16; a tile's sum is multiplied by this.
constexpr float kLevelScale = 16.0f;
// Workgroups that stage activations for all their waves try the fp16 form
// first at every row count (the decode pass at T = 8: 72 % of 8 TB/s
// against 70 % with bf16 levels); a wave that stages its own range converts
// its share itself, which the fp16 form repays up to two rows (5,120 x
// 17,408 split at T = 2: 17.5 us against 20.2 with bf16 levels; 5,120 x
// 5,120 8.0 against 8.3) but not above (at T = 4 8.9 us with bf16 levels
// against 9.2, at T = 8 9.4 against 12.2).
constexpr int kF16MaxT = 16;
constexpr int kF16MaxSplitT = 2;
constexpr int kF16MaxSharedRt4T = 8;
template <int TT, bool SHARED, int RT = 1>
constexpr bool tries_f16() {
  return TT <= (SHARED ? (RT >= 4 ? kF16MaxSharedRt4T : kF16MaxT) : kF16MaxSplitT);
}
// The fp16 form's activations are x * 2^E, first tried with E = kDirectE;
// a tile's sum is multiplied by 2^-E.
constexpr int kDirectE = 4;
constexpr int kNoDirect = 1 << 20;  // no E fits the slice

// 2^e as an fp32 bit pattern (|e| <= 126; for e uniform, scalar arithmetic).
__device__ __forceinline__ float pow2(int e) { return __int_as_float((127 + e) << 23); }

// The E of a slice whose values missed the window of 2^kDirectE, or
// kNoDirect.  x * 2^E is exact in fp16 for every value of 8 significant bits
// from 2^-17 to 65280 (subnormals hold 8 bits down to 2^-17), i.e. for bf16
// magnitude bits b with 0x3700 <= b + 128 E <= 0x477F.  b_max is the
// slice's largest magnitude; mn_min its smallest nonzero magnitude minus 1
// (0xFFFF: no nonzero value).  |E| <= 100 keeps 2^E and 2^-E normal fp32
// numbers.  Of the exponents that fit, the one nearest kDirectE.  No E fits
// an infinity or NaN, a bf16 subnormal, or a span of more than 33 binades.
__device__ __forceinline__ int direct_exponent(unsigned b_max, unsigned mn_min) {
  if (b_max >= 0x7F80u) return kNoDirect;
  const int hi = min(((int)0x477F - (int)b_max) >> 7, 100);        // floor
  const int lo = mn_min >= 0xFFFFu ? -100 : max(-(((int)mn_min + 1 - 0x3700) >> 7), -100);  // ceil
  return lo <= hi ? max(lo, min(kDirectE, hi)) : kNoDirect;
}

__device__ __forceinline__ float bf16_to_f32(unsigned short b) { return __uint_as_float((unsigned)b << 16); }

// Reads through a pointer known to address global memory.  Pointers taken
// from a grouped launch's device table are generic to the compiler, which
// then emits flat loads; those also count against the LDS wait counter, so
// each wait for the staged activations would wait for the weight loads in
// flight too.
template <typename V>
__device__ __forceinline__ V ld_global(const V* p) {
  return *(const __attribute__((address_space(1))) V*)p;
}
template <typename V>
__device__ __forceinline__ V ld_global_nt(const V* p) {
  return __builtin_nontemporal_load((const __attribute__((address_space(1))) V*)p);
}
template <typename V>
__device__ __forceinline__ void st_global(V* p, V v) {
  *(__attribute__((address_space(1))) V*)p = v;
}
// Output store of a kernel for TT activation rows, as each tile completes.
// Up to 4 rows the outputs are written nontemporal, so that fewer dirty
// lines wait in L2 for the write-back at the end of the launch (27B-class
// step at T = 4: +1.0%, body pass at T = 1: +0.3%); from 8 rows on plain
// stores measured faster (T = 8: 0.2%, T = 16: 1.4%).  Run workgroups that
// collect their outputs in LDS write them nontemporal at every row count.
template <int TT>
__device__ __forceinline__ void st_out(float* p, float v) {
  if constexpr (TT <= 4)
    __builtin_nontemporal_store(v, (__attribute__((address_space(1))) float*)p);
  else
    st_global(p, v);
}
// An argmax partial (value bits, id) as one 8-byte store.
__device__ __forceinline__ void st_partial(int2* p, float v, int id) {
  st_global(reinterpret_cast<unsigned long long*>(p),
            (unsigned long long)__float_as_uint(v) | ((unsigned long long)(unsigned)id << 32));
}

// v_cvt_off_f32_i4 on bits 0-3 of byte B of v: the signed nibble n as n / 16.
// The byte is masked out so that the compiler folds its selection into the
// conversion (an SDWA byte select: one instruction per nibble).  No inline
// assembly here or in the other level helpers: the hazard checks that keep
// VALU work clear of in-flight matrix-core results cannot see into it.
template <int B>
__device__ __forceinline__ float nibble_f32(unsigned v) {
  return __builtin_amdgcn_cvt_off_f32_i4(B == 3 ? v >> 24 : (v >> (8 * B)) & 0xFFu);
}

// The value of x, opaque to the optimiser (no instruction): keeps a shifted
// word from being merged into later shifts, and a constant in a register.
__device__ __forceinline__ unsigned opaque_v(unsigned x) {
  asm("" : "+v"(x));
  return x;
}

// The bf16 pair (lo, hi) made of the top halves of two floats.
__device__ __forceinline__ unsigned bf16_pair(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// Eight exact bf16 levels (q - 8) / 16 of one word, in k order.
__device__ __forceinline__ u4_t levels8(unsigned w) {
  const unsigned e = w ^ 0x88888888u;  // even k in bits 0-3 of each byte
  const unsigned o = opaque_v(e >> 4);  // odd k
  return u4_t{bf16_pair(nibble_f32<0>(e), nibble_f32<0>(o)), bf16_pair(nibble_f32<1>(e), nibble_f32<1>(o)),
              bf16_pair(nibble_f32<2>(e), nibble_f32<2>(o)), bf16_pair(nibble_f32<3>(e), nibble_f32<3>(o))};
}

template <typename V>
__device__ __forceinline__ unsigned as_u32(V h) {
  static_assert(sizeof(V) == 4, "packed pair");
  return __builtin_bit_cast(unsigned, h);
}

// The value of x in a scalar register, opaque to the optimiser.
__device__ __forceinline__ unsigned opaque_s(unsigned x) {
  asm("" : "+s"(x));
  return x;
}

// (w & m) | c as one v_and_or_b32: with m and c held in registers (opaque
// to the optimiser, so not folded back into literals, which this VOP3 form
// cannot take) the compiler selects it over an and and an or.
__device__ __forceinline__ unsigned and_or(unsigned w, unsigned m, unsigned c) {
  return (w & opaque_s(m)) | opaque_v(c);
}

// Eight exact fp16 levels (q - 8) of one word, slot order 0,4,1,5,2,6,3,7.
__device__ __forceinline__ u4_t levels8_f16(unsigned w) {
  const unsigned w8 = w >> 8;
  const h2_t lo_bias = {(_Float16)-1032.0f, (_Float16)-1032.0f};
  const h2_t hi_bias = {(_Float16)-72.0f, (_Float16)-72.0f};
  const h2_t a = __builtin_bit_cast(h2_t, and_or(w, 0x000F000Fu, 0x64006400u)) + lo_bias;
  const h2_t b = __builtin_bit_cast(h2_t, and_or(w, 0x00F000F0u, 0x54005400u)) + hi_bias;
  const h2_t c = __builtin_bit_cast(h2_t, and_or(w8, 0x000F000Fu, 0x64006400u)) + lo_bias;
  const h2_t d = __builtin_bit_cast(h2_t, and_or(w8, 0x00F000F0u, 0x54005400u)) + hi_bias;
  return u4_t{as_u32(a), as_u32(b), as_u32(c), as_u32(d)};
}

// One DPP lane move (row-local control; every lane of every row written).
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ unsigned dpp_u32(unsigned v) {
  return (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// Sum over the 32 lanes of each half-wave, every lane receiving the same
// total: within each 16-lane DPP row, row_mirror (lane i with 15 - i), then
// row_half_mirror (i with 7 - i in each half row), then quad_perm xor 2 and
// xor 1, each an add fused with the lane move; then the two rows' totals
// meet through ds_swizzle (xor 16 within 32 lanes).  A fixed order, and by
// symmetry the same value in every lane.
__device__ __forceinline__ float sum32(float v) {
  v += dpp_move<0x140>(v);  // row_mirror
  v += dpp_move<0x141>(v);  // row_half_mirror
  v += dpp_move<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v += dpp_move<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  // ds_swizzle bit mode: and_mask 0x1F, or_mask 0, xor_mask 0x10
  return v + __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
}

// v_dot2_f32_bf16 on two words of packed bf16 pairs: c + a.lo*b.lo + a.hi*b.hi.
__device__ __forceinline__ float dot2(unsigned a, unsigned b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2_t, a), __builtin_bit_cast(b2_t, b), c, false);
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
  const int64_t w = a.row_ids ? (int64_t)ld_global(a.row_ids + o) : o;
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
    if (lane == 0) st_partial(a.partial + wg * TT + t, bv, bi);
  }
}

// ---------------------------------------------------------- staging ----
//
// A staged slice holds token row t at xs + t * xs_stride as a run of 16-byte
// chunks (eight bf16 in k order, 16 chunks per 128-column group).  Chunk c
// of row t sits at position c ^ g(t) of the row, where g keeps bits 0-1 of t
// and swaps bits 2 and 3.  A lane (row r, quarter kq) of the matrix-core
// loop reads chunk 4 kq + j of its row; with g, the 32 lanes of quarters
// 0-1 (or 2-3) over eight token rows read 16 different chunk positions, i.e.
// all 64 LDS banks once, and the 16 lanes of one quarter over sixteen rows
// do the same, so the rows need no padding: T rows of K activations take
// exactly T * K * 2 bytes (T = 16, K = 5120 is a CU's whole 160 KB).  The
// XOR stays inside the aligned 16 chunks of one group.

__device__ __forceinline__ int swz(int t, int c) { return c ^ ((t & 3) | ((t & 4) << 1) | ((t & 8) >> 1)); }

// Stages x[t][gs*128 .. ge*128) of the TT token rows, bf16 as they are, by
// direct global-to-LDS copies (global_load_lds_dwordx4: no registers, no
// conversion).  Wave `wave` of `nwaves` fills 64 consecutive chunk positions
// of one staged row per copy: position p of row t takes chunk swz(t, p) (the
// swizzle is its own inverse).  A staged row holds a multiple of 64 chunk
// positions; positions past the slice (the load ring's padding up to whole
// cycles of eight groups) are written as zeros, which keeps the padded
// slots' products zero (their scale is zero too).  Returns once this
// thread's copies have landed (vmcnt 0, so also every load issued before);
// the caller then makes them visible to the other waves that read them.
template <int TT>
__device__ __forceinline__ void stage_x(const GemvArgs& a, __bf16* xs, int gs, int ge, int wave, int nwaves) {
  const int lane = threadIdx.x & 63;
  const int n = (ge - gs) * (kGroup / 8);  // chunks of the slice per token row
  const int dst_row = a.xs_stride / 8;     // chunk positions per staged row: a multiple of 64
  const int total = TT * dst_row;
  const uint16_t* src = a.x + (int64_t)gs * kGroup;
  unsigned char* lds = reinterpret_cast<unsigned char*>(xs);
  for (int base = wave * 64; base < total; base += nwaves * 64) {
    const int t = base / dst_row;
    const int c = swz(t, base - t * dst_row + lane);
    if (c < n)
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src + (int64_t)t * a.K + c * 8),
                                       (__attribute__((address_space(3))) void*)(lds + (int64_t)base * 16), 16, 0, 0);
    else
      *reinterpret_cast<u4_t*>(lds + (int64_t)(base + lane) * 16) = u4_t{0u, 0u, 0u, 0u};
  }
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
}

// The same staging by one wave through its registers (16-byte loads, four
// in flight per lane, then swizzled LDS stores), for waves that stage their
// own K range.  Such a wave's K loop follows with no workgroup barrier; with
// direct global-to-LDS copies in the kernel the compiler made that loop
// wait for every load in flight at each cycle of the ring (it cannot tell
// the copies have landed), so these kernels copy through registers.
template <int TT>
__device__ __forceinline__ void stage_x_wave(const GemvArgs& a, unsigned char* xs, int gs, int ge) {
  constexpr int kBatch = 4;
  const int lane = threadIdx.x & 63;
  const int n = (ge - gs) * (kGroup / 8);      // chunks of the slice per token row
  const int dst_row = a.xs_stride / 8;         // chunk positions per staged row
  const int total = TT * dst_row;
  const u4_t* src = reinterpret_cast<const u4_t*>(a.x + (int64_t)gs * kGroup);
  u4_t* dst = reinterpret_cast<u4_t*>(xs);
  const int src_row = a.K / 8;
  for (int base = lane; base < total; base += kBatch * 64) {
    u4_t v[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int pos = base + i * 64;
      const int t = pos / dst_row;
      const int c = swz(t, pos - t * dst_row);
      v[i] = (pos < total && c < n) ? ld_global(src + t * src_row + c) : u4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i)
      if (base + i * 64 < total) dst[base + i * 64] = v[i];
  }
}

// ------------------------------------------------------------ fp16 staging ----
//
// The same staged layout with fp16 values times 2^E, each chunk's eight
// values in the fp16 levels' slot order 0,4,1,5,2,6,3,7.

// Eight bf16 (natural order) -> eight fp16 in slot order, scaled by k (a
// power of two); exact for every value inside its window (range_ok for
// 2^kDirectE, direct_exponent for the others).
__device__ __forceinline__ u4_t convert8_f16(u4_t v, float k) {
  const float x0 = __uint_as_float(v.x << 16) * k, x1 = __uint_as_float(v.x & 0xFFFF0000u) * k;
  const float x2 = __uint_as_float(v.y << 16) * k, x3 = __uint_as_float(v.y & 0xFFFF0000u) * k;
  const float x4 = __uint_as_float(v.z << 16) * k, x5 = __uint_as_float(v.z & 0xFFFF0000u) * k;
  const float x6 = __uint_as_float(v.w << 16) * k, x7 = __uint_as_float(v.w & 0xFFFF0000u) * k;
  return u4_t{as_u32(__builtin_amdgcn_cvt_pkrtz(x0, x4)), as_u32(__builtin_amdgcn_cvt_pkrtz(x1, x5)),
              as_u32(__builtin_amdgcn_cvt_pkrtz(x2, x6)), as_u32(__builtin_amdgcn_cvt_pkrtz(x3, x7))};
}

// Running range of the bf16 magnitudes m of eight values: mx = max m, mn =
// min (m - 1) mod 2^16 (a zero wraps to 0xFFFF and never counts as small).
__device__ __forceinline__ void range8(u4_t v, us2_t& mx, us2_t& mn) {
  const us2_t one = {1, 1};
  const unsigned w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const us2_t m = __builtin_bit_cast(us2_t, w[i] & 0x7FFF7FFFu);
    mx = __builtin_elementwise_max(mx, m);
    mn = __builtin_elementwise_min(mn, m - one);
  }
}

// A bf16 times 2^kDirectE converts to fp16 exactly when it is zero or its
// magnitude lies in [2^-21, 4080] (8 significant bits: scaled, fp16 normals
// from 2^-14, subnormals keep 8 bits down to 2^-17, and the largest bf16
// below 2^16 is 65280).  As bf16 magnitude bits: 2^-21 is 0x3500 (mn holds
// m - 1), 4080 is 0x457F.
static_assert(kDirectE == 4, "range_ok's bounds are written for 2^4");
__device__ __forceinline__ bool range_ok(us2_t mx, us2_t mn) {
  return max((unsigned)mx.x, (unsigned)mx.y) <= 0x457Fu && min((unsigned)mn.x, (unsigned)mn.y) >= 0x34FFu;
}

// Zeroes groups [n, next multiple of 8) of every staged row: the load ring
// runs whole cycles of eight groups, and its padded slots read these.
template <int TT>
__device__ __forceinline__ void zero_pad(const GemvArgs& a, unsigned char* xs, int n, int tid, int nthreads) {
  const int b0 = n * (kGroup / 8), b1 = ((n + kRing - 1) / kRing) * kRing * (kGroup / 8);
  const int per_row = b1 - b0;
  if (per_row == 0) return;
  u4_t* dst = reinterpret_cast<u4_t*>(xs);
  const int dst_row = a.xs_stride / 8;
  for (int i = tid; i < TT * per_row; i += nthreads) {
    const int t = i / per_row, b = b0 + i % per_row;
    dst[t * dst_row + swz(t, b)] = u4_t{0u, 0u, 0u, 0u};
  }
}

// fp16 staging of x[t][gs*128 .. ge*128) by threads tid = 0..nthreads-1:
// four 16-byte chunks per thread in flight at a time.  Returns true when
// some value of this thread's chunks is outside the exact window (the
// caller then stages bf16 instead).  A chunk whose position is in
// [hold_from, hold_from + 4) is not stored but returned in held / held_at
// (a thread meets at most one: they are four of one group's 16 chunks and
// nthreads >= 64).
template <int TT>
__device__ __forceinline__ bool stage_direct(const GemvArgs& a, unsigned char* xs, int gs, int ge, int tid,
                                             int nthreads, int hold_from, u4_t& held, int& held_at, float k,
                                             unsigned& b_max, unsigned& mn_min) {
  constexpr int kBatch = 4;
  const int n8 = (ge - gs) * (kGroup / 8);  // chunks per token row
  const int total = TT * n8;
  const u4_t* src = reinterpret_cast<const u4_t*>(a.x + (int64_t)gs * kGroup);
  u4_t* dst = reinterpret_cast<u4_t*>(xs);
  const int src_row = a.K / 8, dst_row = a.xs_stride / 8;
  us2_t mx = {0, 0}, mn = {0xFFFF, 0xFFFF};
  int t = 0, b = tid;  // chunk (t, b) has index t * n8 + b
  while (b >= n8 && t < TT) {
    b -= n8;
    ++t;
  }
  for (int base = tid; base < total; base += kBatch * nthreads) {
    u4_t v[kBatch];
    int d[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      d[i] = t < TT ? t * dst_row + swz(t, b) : -1;
      if (t < TT) v[i] = ld_global(src + t * src_row + b);
      b += nthreads;
      while (b >= n8 && t < TT) {
        b -= n8;
        ++t;
      }
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      if (d[i] >= 0) {
        range8(v[i], mx, mn);
        const u4_t c = convert8_f16(v[i], k);
        if (d[i] >= hold_from) {
          held = c;
          held_at = d[i];
        } else {
          dst[d[i]] = c;
        }
      }
    }
  }
  b_max = max(mx.x, mx.y);
  mn_min = min(mn.x, mn.y);
  return !range_ok(mx, mn);
}

// Largest / smallest value over the wave (uniform).
__device__ __forceinline__ unsigned wave_umax(unsigned v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, (unsigned)__shfl_xor((int)v, o));
  return __builtin_amdgcn_readfirstlane(v);
}
__device__ __forceinline__ unsigned wave_umin(unsigned v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, (unsigned)__shfl_xor((int)v, o));
  return __builtin_amdgcn_readfirstlane(v);
}

// A wave's own staging with its activations loaded ahead of its weights:
// kXPre 16-byte chunks per lane cover T rows of a slice of up to 64 / T
// groups (e.g. the 8-group share of a split wave at K = 5120 up to T = 8).
// Loaded first, they complete first, so the wave stages them and starts
// its first group while its weight loads, issued after them, are still in
// flight (staged after the weights, the wave would wait for all of them).
// Prefetching waves with more than one activation row stage them before
// issuing any weight load: their activation loads then no longer queue
// behind the CU's weight traffic (5,120 x 5,120 at T = 4: 9.0 us against
// 9.9).  A single row is cheaper to wait for behind the weights (8.0 us
// against 8.8 staged first).
template <int TT>
constexpr bool stage_first() { return TT >= 2; }

constexpr int kXPre = 16;

// Row of chunk c (c < 1024) of a slice of n8 chunks per row (n8 <= 1024):
// c * ceil(2^20 / n8) >> 20 is exact while c * n8 < 2^20.
__device__ __forceinline__ int chunk_row(int c, uint32_t inv) { return (int)(__umul24((uint32_t)c, inv) >> 20); }

// Chunk c = lane + 64 i of x[t][gs*128 .. ge*128) (row t = c / n8, chunk
// c % n8 of the row) into xr[i].  Whole instructions past the slice are
// skipped (a uniform test); lanes past its end re-read its last chunk, so
// that every load the wave issues is unconditional.
template <int TT>
__device__ __forceinline__ void prefetch_x(const GemvArgs& a, int gs, int ge, u4_t (&xr)[kXPre]) {
  const int lane = threadIdx.x & 63;
  const int n8 = (ge - gs) * (kGroup / 8), total = TT * n8;
  const uint32_t inv = ((1u << 20) + n8 - 1) / n8;
  const u4_t* src = reinterpret_cast<const u4_t*>(a.x + (int64_t)gs * kGroup);
#pragma unroll
  for (int i = 0; i < kXPre; ++i) {
    if (64 * i < total) {
      const int c = min(lane + 64 * i, total - 1);
      const int t = chunk_row(c, inv);
      xr[i] = ld_global(src + t * (a.K / 8) + (c - t * n8));
    }
  }
}

// Stages the prefetched slice into this wave's LDS area (and the ring
// padding) and returns the level form to run: the fp16 form's fold 2^-E
// when the kernel tries it and some E makes every value exact (kDirectE
// first), else 0 with the bf16 values staged as they are.
template <int TT>
__device__ __forceinline__ float stage_wave_regs(const GemvArgs& a, unsigned char* xs, int gs, int ge,
                                                 const u4_t (&xr)[kXPre]) {
  const int lane = threadIdx.x & 63;
  const int n8 = (ge - gs) * (kGroup / 8), total = TT * n8;
  const uint32_t inv = ((1u << 20) + n8 - 1) / n8;
  const int dst_row = a.xs_stride / 8;
  u4_t* dst = reinterpret_cast<u4_t*>(xs);
  int e = kNoDirect;
  if constexpr (tries_f16<TT, false>()) {
    // lanes past the end hold the last chunk again: harmless to the range
    us2_t mx = {0, 0}, mn = {0xFFFF, 0xFFFF};
#pragma unroll
    for (int i = 0; i < kXPre; ++i)
      if (64 * i < total) range8(xr[i], mx, mn);
    if (__ballot(!range_ok(mx, mn)) == 0)
      e = kDirectE;
    else
      e = direct_exponent(wave_umax(max(mx.x, mx.y)), wave_umin(min(mn.x, mn.y)));
  }
  const bool h = e != kNoDirect;
  const float k = h ? pow2(e) : 0.0f;
#pragma unroll
  for (int i = 0; i < kXPre; ++i) {
    if (64 * i < total) {
      const int c = lane + 64 * i;
      const int t = chunk_row(c, inv);
      if (c < total) dst[t * dst_row + swz(t, c - t * n8)] = h ? convert8_f16(xr[i], k) : xr[i];
    }
  }
  zero_pad<TT>(a, xs, ge - gs, lane, 64);
  return h ? pow2(-e) : 0.0f;
}

// fp16 staging of a slice for the whole workgroup.  Returns (uniform) the
// fp16 form's fold 2^-E when some E makes every value of the slice exact in
// fp16 (kDirectE is tried first; when it misses, the workgroup's range picks
// another and the slice is staged again): the slice and its ring padding
// are then staged.  Otherwise it returns 0, nothing usable is staged and the
// caller stages bf16.  The workgroup-wide decision needs one word per wave;
// the words borrow the last four chunks of the last row, whose values the
// threads that own them hold back until the decision is made.  Ends with a
// barrier after the decision, before any padding store; the caller's barrier
// publishes the staged values.
template <int TT>
__device__ __forceinline__ float stage_f16_shared(const GemvArgs& a, unsigned char* xs, int gs, int ge) {
  const int n8 = (ge - gs) * (kGroup / 8);
  const int flag_at = (TT - 1) * (a.xs_stride / 8) + n8 - 4;  // chunk position of the flag words
  u4_t held = {0u, 0u, 0u, 0u};
  int held_at = -1;
  unsigned b_max, mn_min;
  const bool bad = stage_direct<TT>(a, xs, gs, ge, threadIdx.x, blockDim.x, flag_at, held, held_at,
                                    pow2(kDirectE), b_max, mn_min);
  u4_t* dst = reinterpret_cast<u4_t*>(xs);
  unsigned* flags = reinterpret_cast<unsigned*>(dst + flag_at);  // 16 words: up to 16 waves
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool wave_bad = __ballot(bad) != 0;
  if ((threadIdx.x & 63) == 0) flags[wave] = wave_bad ? 1u : 0u;
  __syncthreads();
  unsigned any = 0;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) any |= flags[i];
  // the same in every lane; said so, the caller's choice of loop is a scalar
  // branch (as a divergent one, both loops' registers would be live at once)
  any = __builtin_amdgcn_readfirstlane(any);
  __syncthreads();  // every wave has read the flags before they are overwritten
  if (any == 0) {
    if (held_at >= 0) dst[held_at] = held;
    zero_pad<TT>(a, xs, ge - gs, threadIdx.x, blockDim.x);
    return pow2(-kDirectE);
  }
  // Some value missed: the workgroup's range, in two of the flag words,
  // picks another power of two if one fits, and the slice is staged again.
  if (threadIdx.x == 0) {
    flags[0] = 0u;
    flags[1] = 0xFFFFFFFFu;
  }
  __syncthreads();
  atomicMax(&flags[0], b_max);
  atomicMin(&flags[1], mn_min);
  __syncthreads();
  const int e = direct_exponent(__builtin_amdgcn_readfirstlane(flags[0]), __builtin_amdgcn_readfirstlane(flags[1]));
  __syncthreads();  // every wave has read the range before the staging overwrites it
  if (e == kNoDirect) return 0.0f;
  stage_direct<TT>(a, xs, gs, ge, threadIdx.x, blockDim.x, 0x7fffffff, held, held_at, pow2(e), b_max, mn_min);
  zero_pad<TT>(a, xs, ge - gs, threadIdx.x, blockDim.x);
  return pow2(-e);
}

// Workgroup staging through registers, for slices of at most kStageRegs
// 16-byte chunks per thread: every chunk load is issued up front, before
// the weight ring, so the activations arrive in one memory round trip that
// overlaps the ring's own instead of queueing behind it in dependent
// batches.  Thread tid holds chunks c = tid + i * nthreads of the slice (row
// t = c / n8, chunk c - t * n8 of the row); threads past the slice's end
// re-read its last chunk (harmless to the range, never stored).
constexpr int kStageRegs = 12;

template <int TT>
__device__ __forceinline__ void prefetch_slice(const GemvArgs& a, int gs, int ge, u4_t (&xr)[kStageRegs]) {
  const int n8 = (ge - gs) * (kGroup / 8), total = TT * n8;
  const int nthreads = blockDim.x;
  const u4_t* src = reinterpret_cast<const u4_t*>(a.x + (int64_t)gs * kGroup);
  int t = 0, b = threadIdx.x;  // t * n8 + b = this thread's chunk c
  while (b >= n8 && t < TT) {
    b -= n8;
    ++t;
  }
#pragma unroll
  for (int i = 0; i < kStageRegs; ++i) {
    if (i * nthreads < total) {  // uniform
      const bool in = t < TT;    // c < total (then b < n8)
      xr[i] = ld_global(src + (in ? t * (a.K / 8) + b : (TT - 1) * (a.K / 8) + n8 - 1));
      b += nthreads;
      while (b >= n8 && t < TT) {
        b -= n8;
        ++t;
      }
    }
  }
}

// Stages the prefetched slice for the whole workgroup (all of its values,
// then the ring padding) and returns the level form to run: the fp16 form's
// fold 2^-E when some E makes every value exact in fp16 (the one nearest
// kDirectE: direct_exponent over the workgroup's range, reduced through two
// LDS words per wave), else 0 with the bf16 values staged as they are.
// Ends before the barrier that publishes the staged values (the caller's).
template <int TT>
__device__ __forceinline__ float stage_regs_shared(const GemvArgs& a, unsigned char* xs, int gs, int ge,
                                                   const u4_t (&xr)[kStageRegs], bool f16) {
  const int n8 = (ge - gs) * (kGroup / 8), total = TT * n8;
  const int nthreads = blockDim.x;
  const int dst_row = a.xs_stride / 8;
  u4_t* dst = reinterpret_cast<u4_t*>(xs);
  int e = kNoDirect;
  if (f16) {
    us2_t mx = {0, 0}, mn = {0xFFFF, 0xFFFF};
#pragma unroll
    for (int i = 0; i < kStageRegs; ++i)
      if (i * nthreads < total) range8(xr[i], mx, mn);
    // the workgroup's range: two words per wave at the start of the staging
    // area (nothing is staged before the decision)
    unsigned* words = reinterpret_cast<unsigned*>(xs);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const unsigned wmax = wave_umax(max(mx.x, mx.y)), wmin = wave_umin(min(mn.x, mn.y));
    if ((threadIdx.x & 63) == 0) {
      words[2 * wave] = wmax;
      words[2 * wave + 1] = wmin;
    }
    __syncthreads();
    unsigned gmax = 0, gmin = 0xFFFFFFFFu;
    for (int w = 0; w < (nthreads >> 6); ++w) {
      gmax = max(gmax, words[2 * w]);
      gmin = min(gmin, words[2 * w + 1]);
    }
    e = direct_exponent(__builtin_amdgcn_readfirstlane(gmax), __builtin_amdgcn_readfirstlane(gmin));
    __syncthreads();  // every wave has read the words before the staging overwrites them
  }
  const bool h = e != kNoDirect;
  const float k = h ? pow2(e) : 0.0f;
  int t = 0, b = threadIdx.x;
  while (b >= n8 && t < TT) {
    b -= n8;
    ++t;
  }
#pragma unroll
  for (int i = 0; i < kStageRegs; ++i) {
    if (i * nthreads < total) {  // uniform
      if (t < TT) dst[t * dst_row + swz(t, b)] = h ? convert8_f16(xr[i], k) : xr[i];
      b += nthreads;
      while (b >= n8 && t < TT) {
        b -= n8;
        ++t;
      }
    }
  }
  zero_pad<TT>(a, xs, ge - gs, threadIdx.x, nthreads);
  return h ? pow2(-e) : 0.0f;
}

// RW rows per wave, L = 64/RW lanes per row; a lane takes the row's 16-byte
// chunks li, li+L, li+2L, ...; CPL bounds the chunks per lane per slice.
// Built for TT <= kDotMaxT (its per-lane sums grow with TT; more rows go to
// the matrix cores).
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
  __bf16* xs = reinterpret_cast<__bf16*>(smem);

  float acc[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) acc[t] = 0.0f;

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
    stage_x<TT>(a, xs, gs, ge, wave, nw);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = li + i * L;
      if (c < nc) {
        const u4_t lv[4] = {levels8(q[i].x), levels8(q[i].y), levels8(q[i].z), levels8(q[i].w)};
        const float sc = bf16_to_f32(sq[i]);
#pragma unroll
        for (int t = 0; t < TT; ++t) {
          const u4_t* xv = reinterpret_cast<const u4_t*>(xs + t * a.xs_stride);
          float p = 0.0f;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const u4_t xw = xv[swz(t, c * 4 + j)];
            p = dot2(lv[j].x, xw.x, p);
            p = dot2(lv[j].y, xw.y, p);
            p = dot2(lv[j].z, xw.z, p);
            p = dot2(lv[j].w, xw.w, p);
          }
          acc[t] = fmaf(p, sc, acc[t]);
        }
      }
    }
  }

  // Sum across the L = 32 lanes of a row (fixed order), with the levels'
  // factor 1/16 taken back first (a power of two: no rounding changes).
  static_assert(L == 32, "the lane reduction covers 32 lanes per row");
#pragma unroll
  for (int t = 0; t < TT; ++t) acc[t] = sum32(acc[t] * kLevelScale);

  float* fin = reinterpret_cast<float*>(smem);  // reused after the last slice
  __syncthreads();
  if (li == 0) {
    const int r = wave * RW + sub;  // row within the workgroup
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      float v = bad ? __builtin_nanf("") : acc[t];
      if (orow < a.n_out && a.y) st_out<TT>(a.y + (int64_t)t * a.n_out + orow, v);
      fin[((r >> 4) * TT + t) * 16 + (r & 15)] = v;
    }
  }
  if (a.partial) {
    __syncthreads();
    if (wave == 0) workgroup_argmax<TT>(a, fin, row0, nw * RW, lane, blockIdx.x);
  }
}

// ---------------------------------------------------------- matrix core ----

// Layout template argument: kLayAny reads either layout (a.tiled decides at
// run time, for grouped launches that mix them); kLayTiled is compiled for
// the tiled layout only, kLayRow for the row-major layout only.
constexpr int kLayAny = 0, kLayTiled = 1, kLayRow = 2;

template <int LAY>
__device__ __forceinline__ bool tiled_rows(const GemvArgs& a) {
  return LAY == kLayTiled || (LAY == kLayAny && a.tiled);
}

// Weight-code load.  kLayAny's row-major loads use the default cache policy:
// its wave load covers 64 bytes of each of 16 rows, and the two 64-byte
// halves of a 128-byte line (groups g and g+1 of a row, loaded by
// consecutive ring slots) then merge into one L2 request in the vector L1,
// which the nontemporal hint would prevent (measured 20% slower).  A tiled
// wave load covers whole lines of a 1 KB block that is read once, and a
// kLayRow wave load whole 128-byte lines of 8 rows: both are marked
// nontemporal (measured 5-9% faster on tiled weights).
template <int LAY>
__device__ __forceinline__ u4_t load_codes(const u4_t* p) {
  if constexpr (LAY == kLayAny)
    return ld_global(p);
  else
    return ld_global_nt(p);
}

// bf16 scale e of eight packed in v (element order = memory order) -> fp32.
__device__ __forceinline__ float scale_of(u4_t v, int e) {
  const unsigned w = (e >> 1) == 0 ? v.x : (e >> 1) == 1 ? v.y : (e >> 1) == 2 ? v.z : v.w;
  return __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
}

// Offset, in 16-byte units, of group g's codes from a lane's code pointer.
template <int LAY>
__device__ __forceinline__ int code_off(const GemvArgs& a, int g) {
  return tiled_rows<LAY>(a) ? (g >> 3) * (kTileChunkBytes / 16) + (g & 7) * (kTileGroupBytes / 16) : 4 * g;
}

// Offset, in 16-byte units, of the eight scales of groups g .. g+7 (g a
// multiple of 8) from a lane's scale pointer.
template <int LAY>
__device__ __forceinline__ int scale_off(const GemvArgs& a, int g) {
  return tiled_rows<LAY>(a)
             ? (g >> 3) * (kTileChunkBytes / 16) + min(kTileChunkGroups, a.G - g) * (kTileGroupBytes / 16)
             : g >> 3;
}


// kLayRow: ring slots 2j and 2j+1 hold the pair of groups (g, g+1), g even.
// The even slot's load reads rows 0-7 of the tile and the odd slot's rows
// 8-15, each as whole 128-byte lines (8 lanes per row: both groups of the
// pair; a plain wave load of one group would cover 16 rows x 64 bytes, half
// lines, which reads HBM at about three quarters of the rate: 5.4 against
// 7.2 TB/s for a plain streaming read of rows 2,560 bytes apart).  In lane
// l (b3 = bit 3 of l, kq = l / 16) the even slot holds row l & 7, group
// g + b3, quarter kq; the odd slot row 8 + (l & 7), group g + 1 - b3.
// pair_groups then hands every lane its own row's (l & 15) quarters of g
// and of g + 1.  cp / cb point at rows l & 7 / 8 + (l & 7) of the tile
// (quarter kq); groups past the row's last are read as its last.
template <int LAY>
__device__ __forceinline__ u4_t load_slot(const GemvArgs& a, const u4_t* cp, const u4_t* cb, int s, int g) {
  if constexpr (LAY == kLayRow) {
    const int b3 = (threadIdx.x >> 3) & 1;
    const int gg = min((g & ~1) + ((s & 1) ? 1 - b3 : b3), a.G - 1);
    return load_codes<LAY>(((s & 1) ? cb : cp) + 4 * gg);
  } else {
    (void)cb;
    (void)s;
    return load_codes<LAY>(cp + code_off<LAY>(a, g));
  }
}

// The exchange after a kLayRow pair of loads (even slot ev, odd slot od):
// lane l's own row l & 15 has group g's quarter in ev (rows 0-7, b3 = 0)
// or od (rows 8-15, b3 = 1) of lane l itself, and group g + 1's in the other
// slot of lane l ^ 8 (a row_ror:8 within the 16-lane DPP row).
__device__ __forceinline__ void pair_groups(const u4_t& ev, const u4_t& od, u4_t& g0, u4_t& g1) {
  const bool b3 = (threadIdx.x >> 3) & 1;
  const u4_t other = b3 ? ev : od;
  g0 = b3 ? od : ev;
  g1 = u4_t{dpp_u32<0x128>(other.x), dpp_u32<0x128>(other.y), dpp_u32<0x128>(other.z), dpp_u32<0x128>(other.w)};
}

// One group of one 16-row tile for this lane: four MFMAs over its four
// words of codes and its four staged activation chunks (xb[j] + group gl);
// H selects the level form (fp16 against the fp16 staging, else bf16).
template <bool H>
__device__ __forceinline__ f4_t group_mfma(const unsigned char* const (&xb)[4], int gl, u4_t w) {
  f4_t d = {0.0f, 0.0f, 0.0f, 0.0f};
  const unsigned ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (H)
      d = __builtin_amdgcn_mfma_f32_16x16x32_f16(*reinterpret_cast<const h8_t*>(xb[j] + gl * (kGroup * 2)),
                                                 __builtin_bit_cast(h8_t, levels8_f16(ww[j])), d, 0, 0, 0);
    else
      d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const b8_t*>(xb[j] + gl * (kGroup * 2)),
                                                  __builtin_bit_cast(b8_t, levels8(ww[j])), d, 0, 0, 0);
    // bf16: one word's levels at a time (the MFMAs chain on d anyway, and
    // forming all four words' levels first would hold 32 more registers);
    // the fp16 levels are cheap enough to interleave freely
    if constexpr (!H) __builtin_amdgcn_sched_barrier(0);
  }
  return d;
}

// This lane's four activation chunks of group 0 of a staged slice (row trow,
// chunks 4 kq .. 4 kq + 3 of the group, swizzled), as byte pointers.
__device__ __forceinline__ void lane_chunks(const GemvArgs& a, const unsigned char* xs, int trow, int kq,
                                            const unsigned char* (&xb)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) xb[j] = xs + (trow * a.xs_stride + swz(trow, kq * 4 + j) * 8) * 2;
}

// Stages the slice [sb, se) of the activations for a workgroup (SHARED) or
// for this wave alone, and returns which level form runs on it: the fp16
// form's fold 2^-E when the kernel tries it (F16, from tries_f16) and some
// power of two 2^E makes every value exact in fp16 (2^kDirectE first), else
// 0 with the bf16 values staged.  Returns after the staged values are
// visible to every wave that reads them and every load issued before has
// landed.
template <int TT, bool SHARED, bool F16>
__device__ __forceinline__ float stage_slice(const GemvArgs& a, unsigned char* xs, int sb, int se) {
  float fold = 0.0f;
  if constexpr (SHARED) {
    if constexpr (F16) fold = stage_f16_shared<TT>(a, xs, sb, se);
    if (fold == 0.0f)
      stage_x<TT>(a, reinterpret_cast<__bf16*>(xs), sb, se, __builtin_amdgcn_readfirstlane(threadIdx.x >> 6),
                  blockDim.x >> 6);
    __syncthreads();
  } else {
    const int lane = threadIdx.x & 63;
    lds_fence();
    if constexpr (F16) {
      u4_t held;
      int held_at = -1;
      unsigned b_max, mn_min;
      int e = kDirectE;
      if (__ballot(stage_direct<TT>(a, xs, sb, se, lane, 64, 0x7fffffff, held, held_at, pow2(kDirectE), b_max,
                                    mn_min)) != 0) {
        // some value missed: the wave's range picks another power of two
        e = direct_exponent(wave_umax(b_max), wave_umin(mn_min));
        if (e != kNoDirect) {
          lds_fence();
          stage_direct<TT>(a, xs, sb, se, lane, 64, 0x7fffffff, held, held_at, pow2(e), b_max, mn_min);
        }
      }
      if (e != kNoDirect) {
        zero_pad<TT>(a, xs, se - sb, lane, 64);
        fold = pow2(-e);
      } else {
        lds_fence();
      }
    }
    if (fold == 0.0f) stage_x_wave<TT>(a, xs, sb, se);
    lds_fence();
  }
  // the staging waited for its loads, issued after the weight loads in
  // flight; saying so lets the loop wait for exactly one group at a time
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  return fold;
}

// The tiles of one staged slice (n groups from sb, np = n rounded up to
// whole ring cycles): the wave streams tile 0's groups, then tile 1's, ...
// with the load ring running across tile boundaries; the ring (q, sq, sv)
// holds tile 0's first groups on entry.  cb: the second row pointers of
// kLayRow (unused otherwise).
template <int TT, int RT, bool VS, int LAY, bool H>
__device__ __forceinline__ void slice_tiles(const GemvArgs& a, const u4_t* const (&cp)[RT],
                                            const u4_t* const (&cb)[RT], const uint16_t* const (&sp)[RT],
                                            const unsigned char* const (&xb)[4], int sb, int n, int np,
                                            u4_t (&q)[kRing], unsigned short (&sq)[kRing], u4_t& sv, float fold,
                                            float (&acc)[RT][4]) {
  constexpr int PD = kRing;
  static_assert(PD % 2 == 0, "kLayRow loads pairs of ring slots");
#pragma unroll
  for (int tl = 0; tl < RT; ++tl) {
    // the ring runs on into the next tile; the last tile's final cycle
    // reloads nothing, so that no load is left in flight past the slice
    const u4_t* cpn = cp[tl + 1 < RT ? tl + 1 : tl];
    const u4_t* cbn = cb[tl + 1 < RT ? tl + 1 : tl];
    const uint16_t* spn = sp[tl + 1 < RT ? tl + 1 : tl];
    const bool has_next = tl + 1 < RT;
    float accs[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    auto cycle = [&](int fi, auto reload) {
      constexpr bool R = decltype(reload)::value;
      const bool last = fi + PD >= np;  // uniform: this cycle prefetches the next tile
      u4_t svn;
      if constexpr (VS && R) {
        const uint16_t* base = (last && has_next) ? spn : sp[tl];
        const int gv = last ? (has_next ? sb : sb + fi) : sb + fi + PD;
        svn = ld_global(reinterpret_cast<const u4_t*>(base) + scale_off<LAY>(a, gv));
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (LAY == kLayRow) {
#pragma unroll
        for (int s = 0; s < PD; s += 2) {
          const int gl = fi + s;  // groups past n read the zeroed padding
          float sc0, sc1;
          if constexpr (VS) {
            sc0 = scale_of(sv, s);
            sc1 = scale_of(sv, s + 1);
          } else {
            sc0 = bf16_to_f32(sq[s]);
            sc1 = bf16_to_f32(sq[s + 1]);
          }
          sc0 = (gl < n) ? sc0 : 0.0f;
          sc1 = (gl + 1 < n) ? sc1 : 0.0f;
          u4_t w0, w1;
          pair_groups(q[s], q[s + 1], w0, w1);
          if constexpr (R) {
            // reload the pair's slots with the groups PD positions ahead
            const int tgt = gl + PD;
            const bool nxt = tgt >= np;
            const bool on = nxt && has_next;
            const int gg = sb + (nxt ? (has_next ? min(tgt - np, n - 1) : n - 1) : min(tgt, n - 1));
            if constexpr (!VS) {
              sq[s] = ld_global((on ? spn : sp[tl]) + gg);
              sq[s + 1] = ld_global((on ? spn : sp[tl]) + min(gg + 1, a.G - 1));
            }
            q[s] = load_slot<LAY>(a, on ? cpn : cp[tl], on ? cbn : cb[tl], s, gg);
            q[s + 1] = load_slot<LAY>(a, on ? cpn : cp[tl], on ? cbn : cb[tl], s + 1, gg);
            __builtin_amdgcn_sched_barrier(0);
          }
          const f4_t d0 = group_mfma<H>(xb, gl, w0);
#pragma unroll
          for (int r = 0; r < 4; ++r) accs[r] = fmaf(d0[r], sc0, accs[r]);
          const f4_t d1 = group_mfma<H>(xb, gl + 1, w1);
#pragma unroll
          for (int r = 0; r < 4; ++r) accs[r] = fmaf(d1[r], sc1, accs[r]);
        }
      } else {
#pragma unroll
        for (int s = 0; s < PD; ++s) {
          const int gl = fi + s;  // groups past n read the zeroed padding
          float sc;
          if constexpr (VS)
            sc = scale_of(sv, s);
          else
            sc = bf16_to_f32(sq[s]);
          sc = (gl < n) ? sc : 0.0f;
          const f4_t d = group_mfma<H>(xb, gl, q[s]);
#pragma unroll
          for (int r = 0; r < 4; ++r) accs[r] = fmaf(d[r], sc, accs[r]);
          if constexpr (R) {
            // reload this slot with the group PD positions ahead
            const int tgt = gl + PD;
            const bool nxt = tgt >= np;
            const u4_t* cpl = (nxt && has_next) ? cpn : cp[tl];
            const int gg = sb + (nxt ? (has_next ? min(tgt - np, n - 1) : n - 1) : min(tgt, n - 1));
            if constexpr (!VS) sq[s] = ld_global(((nxt && has_next) ? spn : sp[tl]) + gg);
            q[s] = load_codes<LAY>(cpl + code_off<LAY>(a, gg));
            // keep this slot's reload here: sunk to the end of the loop, the
            // reloads would make every iteration wait for the whole ring
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      if constexpr (VS && R) sv = svn;
    };
    const int reloading = has_next ? np : np - PD;  // cycles that reload their slots
    int fi = 0;
    for (; fi < reloading; fi += PD) cycle(fi, std::true_type{});
    if (!has_next) cycle(fi, std::false_type{});
    // fold this tile's slice sum, undoing the level form's power of two
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[tl][r] += accs[r] * fold;
  }
}

// The exact fallback of the kernels that try the fp16 form: groups
// [g0, g0 + n) of one tile, one group at a time with bf16 levels against
// the bf16 staging (xb: this lane's chunks of the staged slice's group 0),
// added into accs.  A short loop with no load ring: it holds few registers,
// so it leaves the fast loop's register allocation alone, and it runs only
// for a slice holding an activation outside the fp16 window.
template <int LAY>
__device__ __forceinline__ void exact_groups(const GemvArgs& a, const u4_t* cp, const uint16_t* sp,
                                             const unsigned char* const (&xb)[4], int g0, int n, float (&accs)[4]) {
  for (int g = 0; g < n; ++g) {
    const int gg = g0 + g;
    const u4_t w = load_codes<LAY>(cp + code_off<LAY>(a, gg));
    // scale of group gg: in its 8-scale block (tiled), or the row's gg-th
    const int si = tiled_rows<LAY>(a) ? scale_off<LAY>(a, gg & ~7) * 8 + (gg & 7) : gg;
    const float sc = bf16_to_f32(ld_global(sp + si));
    const f4_t d = group_mfma<false>(xb, g, w);
#pragma unroll
    for (int r = 0; r < 4; ++r) accs[r] = fmaf(d[r], sc, accs[r]);
  }
}

template <int TT, int RT, int LAY>
__device__ __forceinline__ void exact_slice(const GemvArgs& a, const u4_t* const (&cp)[RT],
                                            const u4_t* const (&cb)[RT], const uint16_t* const (&sp)[RT],
                                            const unsigned char* const (&xb)[4], int sb, int n, float (&acc)[RT][4]) {
  // kLayRow: this lane's own row (l & 15) is row l & 7 of cp or 8 + (l & 7) of cb
  const bool own_b = LAY == kLayRow && ((threadIdx.x >> 3) & 1);
#pragma unroll
  for (int tl = 0; tl < RT; ++tl) {
    float accs[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    exact_groups<LAY>(a, own_b ? cb[tl] : cp[tl], sp[tl], xb, sb, n, accs);
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[tl][r] += accs[r] * kLevelScale;
  }
}

// The K loop of one wave: groups [g_begin, g_end) of RT 16-row tiles.  The
// range is cut into slices that fit the staged activations; within a slice
// the wave streams tile 0's groups, then tile 1's, ... with kRing groups of
// codes in flight and the ring running across tile boundaries.  A lane owns
// output row r16 of a tile and quarter kq of each 128-column group: one
// 16-byte load per group feeds four MFMAs (tokens as the A operand, padded to
// 16 rows; weights as the B operand), whose sum gets the group's scale.
// SHARED: the slice is staged once for the whole workgroup; otherwise each
// wave stages its own range (no barrier).
// VS: scales are read eight groups (16 bytes) per load (needs G % 8 == 0,
// 16-byte aligned scale rows and g_begin % 8 == 0); otherwise one 2-byte
// load per group.
template <int TT, int RT, bool VS, bool SHARED, int LAY, bool PRE>
__device__ __forceinline__ void stream_slice(const GemvArgs& a, const u4_t* const (&cp)[RT],
                                             const u4_t* const (&cb)[RT], const uint16_t* const (&sp)[RT],
                                             unsigned char* xs, int sb, int se, bool first, int trow, int kq,
                                             float (&acc)[RT][4]) {
  constexpr int PD = kRing;
  u4_t q[PD];
  unsigned short sq[PD];
  u4_t sv;
  const int n = se - sb;                  // groups of this slice
  const int np = (n + PD - 1) / PD * PD;  // padded to whole ring cycles
  // Ring prologue (tile 0 of the slice): slot order, as the loop reloads them.
  auto prologue = [&]() {
    if constexpr (VS) sv = ld_global(reinterpret_cast<const u4_t*>(sp[0]) + scale_off<LAY>(a, sb));
#pragma unroll
    for (int s = 0; s < PD; ++s) {
      const int g = sb + min(s, n - 1);
      if constexpr (!VS) sq[s] = ld_global(sp[0] + g);
      q[s] = load_slot<LAY>(a, cp[0], cb[0], s, g);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  float fold;  // the fp16 form's 2^-E, or 0: bf16 staged
  if constexpr (PRE) {
    // the wave's activations are loaded first, into registers
    u4_t xr[kXPre];
    prefetch_x<TT>(a, sb, se, xr);
    if constexpr (!stage_first<TT>()) prologue();
    lds_fence();
    fold = stage_wave_regs<TT>(a, xs, sb, se, xr);
    lds_fence();
    if constexpr (stage_first<TT>()) prologue();
  } else {
    // issued before the activations are staged, so that the weight latency
    // overlaps the activation round trip
    prologue();
    if constexpr (SHARED)
      if (!first) __syncthreads();  // every wave is done with the previous slice
    fold = stage_slice<TT, SHARED, tries_f16<TT, SHARED, RT>()>(a, xs, sb, se);
  }
  const unsigned char* xb[4];
  lane_chunks(a, xs, trow, kq, xb);
  if constexpr (tries_f16<TT, SHARED, RT>()) {
    if (fold != 0.0f)
      slice_tiles<TT, RT, VS, LAY, true>(a, cp, cb, sp, xb, sb, n, np, q, sq, sv, fold, acc);
    else
      exact_slice<TT, RT, LAY>(a, cp, cb, sp, xb, sb, n, acc);
  } else {
    (void)fold;
    slice_tiles<TT, RT, VS, LAY, false>(a, cp, cb, sp, xb, sb, n, np, q, sq, sv, kLevelScale, acc);
  }
}

// The slices of [g_begin, g_end) in turn.  A wave staging its own range (not
// SHARED) in one slice that fits kXPre loads per lane takes the prefetching
// form: its activations are loaded ahead of its weights and staged as soon
// as they land, while the weights are still in flight.
template <int TT, int RT, bool VS, bool SHARED, int LAY>
__device__ __forceinline__ void stream_tiles(const GemvArgs& a, const u4_t* const (&cp)[RT],
                                             const u4_t* const (&cb)[RT], const uint16_t* const (&sp)[RT],
                                             unsigned char* xs, int g_begin, int g_end, int trow, int kq,
                                             float (&acc)[RT][4]) {
  if constexpr (!SHARED && TT <= 8) {
    if (g_end - g_begin <= a.sk && TT * (g_end - g_begin) * (kGroup / 8) <= kXPre * 64) {  // uniform
      stream_slice<TT, RT, VS, SHARED, LAY, true>(a, cp, cb, sp, xs, g_begin, g_end, true, trow, kq, acc);
      return;
    }
  }
  for (int sb = g_begin; sb < g_end; sb += a.sk)
    stream_slice<TT, RT, VS, SHARED, LAY, false>(a, cp, cb, sp, xs, sb, min(g_end, sb + a.sk), sb == g_begin,
                                                 trow, kq, acc);
}

// Code and scale pointers of the RT tiles starting at output row row0 for
// this lane.  Row-major: the row's codes (quarter kq) and scales.  Tiled:
// the lane's 16 bytes in the first group block of the row's tile, and the
// row's 16 bytes in the first scale block.  kLayRow: cp and cb point at the
// codes (quarter kq) of rows l & 7 and 8 + (l & 7) of the tile, one of which
// is the lane's own row l & 15; sp at its own row's scales.  Elsewhere cb =
// cp.
template <int RT, int LAY>
__device__ __forceinline__ void tile_pointers(const GemvArgs& a, int64_t row0, int r16, int kq,
                                              const u4_t* (&cp)[RT], const u4_t* (&cb)[RT],
                                              const uint16_t* (&sp)[RT]) {
  const int64_t kh = a.K >> 1;
#pragma unroll
  for (int tl = 0; tl < RT; ++tl) {
    if constexpr (LAY == kLayRow) {
      const int64_t r0 = row0 + tl * 16 + (r16 & 7);
      int64_t wa = weight_row(a, r0), wb = weight_row(a, r0 + 8);
      wa = wa < 0 ? 0 : wa;  // read a valid row; the output is masked later
      wb = wb < 0 ? 0 : wb;
      cp[tl] = reinterpret_cast<const u4_t*>(a.packed + wa * kh) + kq;
      cb[tl] = reinterpret_cast<const u4_t*>(a.packed + wb * kh) + kq;
      sp[tl] = a.scales + (r16 >= 8 ? wb : wa) * a.G;
      continue;
    }
    int64_t w = weight_row(a, row0 + tl * 16 + r16);
    if (w < 0) w = 0;  // read a valid row; the output is masked later
    if (tiled_rows<LAY>(a)) {
      const uint8_t* tb = a.packed + (w >> 4) * a.tile_bytes;
      cp[tl] = reinterpret_cast<const u4_t*>(tb) + 4 * (w & 15) + kq;
      sp[tl] = reinterpret_cast<const uint16_t*>(tb) + 8 * (w & 15);
    } else {
      cp[tl] = reinterpret_cast<const u4_t*>(a.packed + w * kh) + kq;
      sp[tl] = a.scales + w * a.G;
    }
    cb[tl] = cp[tl];
  }
}

// Split workgroup: its a.nw waves own the same RT tiles (rows wg*16*RT ..) and
// split K into ranges of a.gpw groups; each wave stages its own range; the
// partial sums are added through LDS in wave order.
template <int TT, int RT, int LAY>
__device__ __forceinline__ void split_workgroup(const GemvArgs& a, int64_t wg, unsigned char* smem) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, kq = lane >> 4;
  const int trow = min(r16, TT - 1);  // A rows >= TT only feed D rows that are never read
  const int64_t row0 = wg * (RT * 16);
  const u4_t* cp[RT];
  const u4_t* cb[RT];
  const uint16_t* sp[RT];
  tile_pointers<RT, LAY>(a, row0, r16, kq, cp, cb, sp);
  const int g_begin = wave * a.gpw;
  const int g_end = (wave < a.nw) ? min(a.G, g_begin + a.gpw) : g_begin;  // uniform
  unsigned char* xs = smem + wave * a.wave_lds;

  float acc[RT][4];
#pragma unroll
  for (int tl = 0; tl < RT; ++tl)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[tl][r] = 0.0f;
  if (g_end > g_begin) {
    if (LAY == kLayTiled || a.vec_scales)
      stream_tiles<TT, RT, true, false, LAY>(a, cp, cb, sp, xs, g_begin, g_end, trow, kq, acc);
    else if constexpr (LAY != kLayTiled)
      stream_tiles<TT, RT, false, false, LAY>(a, cp, cb, sp, xs, g_begin, g_end, trow, kq, acc);
  }

  // Split-K partials of this wave -> its own LDS area: red[(tl*TT + t)*16 + row].
  lds_fence();
  float* red = reinterpret_cast<float*>(smem + wave * a.wave_lds);
  if (wave < a.nw) {
#pragma unroll
    for (int tl = 0; tl < RT; ++tl)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = kq * 4 + r;
        if (t < TT) red[(tl * TT + t) * 16 + r16] = acc[tl][r];
      }
  }
  __syncthreads();

  // The final values overwrite wave 0's partials: output o is read (all
  // waves) and then written by one thread only.
  float* fin = reinterpret_cast<float*>(smem);
  constexpr int kOut = RT * TT * 16;
  for (int o = threadIdx.x; o < kOut; o += blockDim.x) {
    float v = 0.0f;
    for (int w = 0; w < a.nw; ++w) v += reinterpret_cast<const float*>(smem + w * a.wave_lds)[o];
    const int tl = o / (TT * 16), t = (o >> 4) % TT, r = o & 15;
    const int64_t orow = row0 + tl * 16 + r;
    if (orow < a.n_out) {
      if (weight_row(a, orow) < 0) v = __builtin_nanf("");
      if (a.y) st_out<TT>(a.y + (int64_t)t * a.n_out + orow, v);
    }
    fin[o] = v;
  }
  if (a.partial) {
    __syncthreads();
    if (wave == 0) workgroup_argmax<TT>(a, fin, row0, RT * 16, lane, wg);
  }
}

// Shared workgroup: each of its waves owns RT tiles of its own over all of K
// (rows (wg*waves + wave)*16*RT ..); the waves share one staged copy of the
// activations per K slice, so the staging is paid once per 16 * RT * waves
// rows.  Every output is summed by one wave.  grouped: the workgroup is one
// of a grouped launch (its outputs may go through LDS, below).
template <int TT, int RT, int LAY>
__device__ __forceinline__ void shared_workgroup(const GemvArgs& a, int64_t wg, unsigned char* smem, bool grouped) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nwv = blockDim.x >> 6;
  const int r16 = lane & 15, kq = lane >> 4;
  const int trow = min(r16, TT - 1);
  const int64_t row_w = (wg * nwv + wave) * (int64_t)(RT * 16);  // first row of this wave
  const u4_t* cp[RT];
  const u4_t* cb[RT];
  const uint16_t* sp[RT];
  tile_pointers<RT, LAY>(a, row_w, r16, kq, cp, cb, sp);
  unsigned char* xs = smem;

  float acc[RT][4];
#pragma unroll
  for (int tl = 0; tl < RT; ++tl)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[tl][r] = 0.0f;
  if (LAY == kLayTiled || a.vec_scales)
    stream_tiles<TT, RT, true, true, LAY>(a, cp, cb, sp, xs, 0, a.G, trow, kq, acc);
  else if constexpr (LAY != kLayTiled)
    stream_tiles<TT, RT, false, true, LAY>(a, cp, cb, sp, xs, 0, a.G, trow, kq, acc);

  float bv[TT];
  int bi[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    bv[t] = __builtin_nanf("");
    bi[t] = -1;
  }
  // In a grouped launch, from two token rows, the workgroup's outputs go
  // through the staging area, free once every wave is done, when it holds
  // them (T x 16 * RT * waves fp32, output (row q of the workgroup's rows,
  // token row t) at q * TT + t; the staging area holds T * xs_stride bf16),
  // and are written token row by token row, as a run workgroup writes its
  // collected block (grouped body pass: +0.3 to +0.9 points at T = 2-8, bit
  // for bit the same results; at T = 1 no gain).  Otherwise each lane stores
  // its own: a single launch's workgroups all end together, and the extra
  // barrier and round trip lengthen its tail (34,816 x 5,120 at T = 4 and
  // 8: +0.3 and +0.7 us).
  const bool collect = grouped && TT >= 2 && a.y && nwv * RT * 32 <= a.xs_stride;  // uniform
  float* const block = reinterpret_cast<float*>(smem);
  if (collect) __syncthreads();  // the staged activations are no longer read
#pragma unroll
  for (int tl = 0; tl < RT; ++tl) {
    const int64_t orow = row_w + tl * 16 + r16;
    const bool in_range = orow < a.n_out;
    const int64_t wr = in_range ? weight_row(a, orow) : -1;
    const bool bad = in_range && wr < 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = kq * 4 + r;
      const float out = bad ? __builtin_nanf("") : acc[tl][r];
      if (collect) {
        if (t < TT) block[((wave * RT + tl) * 16 + r16) * TT + t] = out;  // rows past n_out: never written out
      } else if (t < TT && in_range && a.y) {
        st_out<TT>(a.y + (int64_t)t * a.n_out + orow, out);
      }
    }
    if (a.partial) {
      // this lane's candidate for token rows t = 4*kq + r
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        const int r = t & 3;
        float v = acc[tl][0];
#pragma unroll
        for (int i = 1; i < 4; ++i) v = (r == i) ? acc[tl][i] : v;
        const int id = (kq == (t >> 2) && wr >= 0 && !__builtin_isnan(v)) ? (int)wr : -1;
        if (better(v, id, bv[t], bi[t])) {
          bv[t] = v;
          bi[t] = id;
        }
      }
    }
  }
  if (collect) {
    __syncthreads();
    const int64_t row0 = wg * nwv * (int64_t)(RT * 16);  // < n_out: the grid holds no empty workgroup
    const int nr = (int)min((int64_t)(nwv * RT * 16), a.n_out - row0);
    for (int t = 0; t < TT; ++t)
      for (int i = threadIdx.x; i < nr; i += (int)blockDim.x)
        __builtin_nontemporal_store(block[i * TT + t],
                                    (__attribute__((address_space(1))) float*)(a.y + (int64_t)t * a.n_out + row0 + i));
  }
  if (a.partial) {
    // per t: best (value, id) of this wave's rows, then of the workgroup
    int2* fin = reinterpret_cast<int2*>(smem);
    __syncthreads();  // the staging area (and the output block) is free now
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      float v = bv[t];
      int id = bi[t];
      wave_argmax(v, id);
      if (lane == 0) fin[wave * TT + t] = int2{__float_as_int(v), id};
    }
    __syncthreads();
    if (wave == 0 && lane < TT) {
      float b = __builtin_nanf("");
      int i = -1;
      for (int w2 = 0; w2 < nwv; ++w2) {
        const int2 c = fin[w2 * TT + lane];
        if (better(__int_as_float(c.x), c.y, b, i)) {
          b = __int_as_float(c.x);
          i = c.y;
        }
      }
      st_partial(a.partial + wg * TT + lane, b, i);
    }
  }
}

// ------------------------------------------------------------- tile runs ----

// The K loop of one wave over a run of whole tiles: v, v + step, ... (< v_end),
// one tile at a time over all of K (one staged slice), with the ring running
// from each tile into the next, so a workgroup pays its start (activation
// staging, ring fill) once for several tiles per wave.  Eight scales per load.
// The caller issued the first tile's ring (ring_prologue with cp, sp).  Each
// tile's outputs are written when its last group is done; with a.partial
// set, the lane keeps its best (value, id) for token rows t = 4 kq + r in
// bv[r] / bi[r].

// Code and scale pointers of tile v (rows 16v .. 16v+15) for this lane; returns
// the lane's weight row (-1: past the end or an invalid id).  kLayRow: cp and
// cb point at rows l & 7 and 8 + (l & 7) of the tile (tile_pointers); else
// cb = cp.
template <int LAY>
__device__ __forceinline__ int tile_ptr(const GemvArgs& a, int64_t v, int r16, int kq, const u4_t*& cp,
                                        const u4_t*& cb, const uint16_t*& sp) {
  if constexpr (LAY == kLayRow) {
    const int64_t r0 = v * 16 + (r16 & 7);
    const int64_t wa_out = weight_row(a, r0), wb_out = weight_row(a, r0 + 8);
    const int64_t wa = wa_out < 0 ? 0 : wa_out, wb = wb_out < 0 ? 0 : wb_out;  // valid rows; outputs masked
    const int64_t kh = a.K >> 1;
    cp = reinterpret_cast<const u4_t*>(a.packed + wa * kh) + kq;
    cb = reinterpret_cast<const u4_t*>(a.packed + wb * kh) + kq;
    sp = a.scales + (r16 >= 8 ? wb : wa) * a.G;
    return (int)(r16 >= 8 ? wb_out : wa_out);
  }
  const int64_t w_out = weight_row(a, v * 16 + r16);
  const int64_t w = w_out < 0 ? 0 : w_out;  // read a valid row; the output is masked
  if (tiled_rows<LAY>(a)) {
    const uint8_t* tb = a.packed + (w >> 4) * a.tile_bytes;
    cp = reinterpret_cast<const u4_t*>(tb) + 4 * (w & 15) + kq;
    sp = reinterpret_cast<const uint16_t*>(tb) + 8 * (w & 15);
  } else {
    cp = reinterpret_cast<const u4_t*>(a.packed + w * (int64_t)(a.K >> 1)) + kq;
    sp = a.scales + w * a.G;
  }
  cb = cp;
  return (int)w_out;
}

// The first ring cycle of a tile over groups [sb, sb + n) (sb a multiple of
// eight): its eight scales and its first eight groups.
template <int LAY>
__device__ __forceinline__ void ring_prologue(const GemvArgs& a, const u4_t* cp, const u4_t* cb, const uint16_t* sp,
                                              int sb, int n, u4_t (&q)[kRing], u4_t& sv) {
  sv = ld_global(reinterpret_cast<const u4_t*>(sp) + scale_off<LAY>(a, sb));
#pragma unroll
  for (int s = 0; s < kRing; ++s) {
    q[s] = load_slot<LAY>(a, cp, cb, s, sb + min(s, n - 1));
    __builtin_amdgcn_sched_barrier(0);  // issue in slot order, as the loop reloads them
  }
}

// Where a run workgroup's outputs go: with `lane` null straight to y as
// each tile completes; otherwise into the workgroup's LDS block, output
// (row 16 (v - v_base) + r, token row t) at block[row * TT + t], which the
// workgroup writes to y at its end.  `lane` is this lane's slot of tile
// v_base, block + r16 * TT + 4 kq: one address register, each tile's four
// stores at fixed offsets from it.  A run over K in slices carries its
// partial sums there: the first slice writes them, later ones add theirs,
// and the last one's sums are the outputs.
struct RunOut {
  float* lane;
  int64_t v_base;
  bool first, last;
};

// Tile v done: this lane's outputs (row 16 v + r16, token rows t = 4 kq + r,
// the tile's sums accs times fold) are stored or collected, and the lane's
// running argmax candidates bv[r] / bi[r] updated when the launch takes the
// argmax.
template <int TT>
__device__ __forceinline__ void tile_outputs(const GemvArgs& a, int64_t v, int r16, int kq, int w_cur,
                                             const float (&accs)[4], float fold, float (&bv)[4], int (&bi)[4],
                                             const RunOut& ro) {
  const int64_t orow = v * 16 + r16;
  const bool in_range = orow < a.n_out;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = kq * 4 + r;
    const float val = accs[r] * fold;  // the level form's power of two undone
    float out = w_cur < 0 ? __builtin_nanf("") : val;
    if (ro.lane) {
      if (t < TT) {  // rows past n_out: never written out
        float* slot = ro.lane + (int)(v - ro.v_base) * (16 * TT) + r;
        if (!ro.first) out = *slot + out;  // the earlier slices' sum, then this one's: their order fixed
        *slot = out;
      }
    } else if (t < TT && in_range && a.y) {
      st_out<TT>(a.y + (int64_t)t * a.n_out + orow, out);
    }
    if (a.partial && ro.last && t < TT && w_cur >= 0 && !__builtin_isnan(out) && better(out, w_cur, bv[r], bi[r])) {
      bv[r] = out;
      bi[r] = w_cur;
    }
  }
}

// The exact fallback of run_tiles (see exact_groups): tiles v, v + step, ...
// (< v_end), groups [sb, sb + n) each, one group at a time.
template <int TT, int LAY>
__device__ __forceinline__ void exact_run_tiles(const GemvArgs& a, int64_t v, int64_t v_end, int step,
                                                const unsigned char* xs, int r16, int kq, int trow, int sb, int n,
                                                float (&bv)[4], int (&bi)[4], const RunOut& ro) {
  const unsigned char* xb[4];
  lane_chunks(a, xs, trow, kq, xb);
  // kLayRow: this lane's own row is row l & 7 of cp or 8 + (l & 7) of cb
  const bool own_b = LAY == kLayRow && r16 >= 8;
  for (; v < v_end; v += step) {  // uniform
    const u4_t* cp;
    const u4_t* cb;
    const uint16_t* sp;
    const int w_cur = tile_ptr<LAY>(a, v, r16, kq, cp, cb, sp);
    float accs[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    exact_groups<LAY>(a, own_b ? cb : cp, sp, xb, sb, n, accs);
    tile_outputs<TT>(a, v, r16, kq, w_cur, accs, kLevelScale, bv, bi, ro);
  }
}

// Tiles v, v + step, ... (< v_end) over groups [sb, sb + n) of K (the staged
// slice; sb a multiple of eight), the ring running from each tile into the
// next; the caller issued the first tile's ring (ring_prologue).
template <int TT, int LAY, bool H>
__device__ __forceinline__ void run_tiles(const GemvArgs& a, int64_t v, int64_t v_end, int step,
                                          const unsigned char* xs, int r16, int kq, int trow, int sb, int n,
                                          const u4_t* cp, const u4_t* cb, const uint16_t* sp, u4_t (&q)[kRing],
                                          u4_t& sv, float fold, float (&bv)[4], int (&bi)[4], const RunOut& ro) {
  constexpr int PD = kRing;
  const int np = (n + PD - 1) / PD * PD;
  const unsigned char* xb[4];  // this lane's activation chunks of group 0
  lane_chunks(a, xs, trow, kq, xb);
  int w_cur = (int)weight_row(a, v * 16 + r16);
  while (v < v_end) {  // uniform
    const int64_t vn = v + step;
    const bool has_next = vn < v_end;
    const u4_t* cpn = cp;
    const u4_t* cbn = cb;
    const uint16_t* spn = sp;
    int w_next = -1;
    if (has_next) w_next = tile_ptr<LAY>(a, vn, r16, kq, cpn, cbn, spn);
    float accs[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int fi = 0; fi < np; fi += PD) {
      const bool last = fi + PD >= np;  // uniform: this cycle prefetches the next tile
      const uint16_t* sbase = (last && has_next) ? spn : sp;
      const int gv = last ? (has_next ? 0 : fi) : fi + PD;
      const u4_t svn = ld_global(reinterpret_cast<const u4_t*>(sbase) + scale_off<LAY>(a, sb + gv));
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (LAY == kLayRow) {
#pragma unroll
        for (int s = 0; s < PD; s += 2) {
          const int gl = fi + s;  // groups past n read the zeroed padding
          const float sc0 = (gl < n) ? scale_of(sv, s) : 0.0f;
          const float sc1 = (gl + 1 < n) ? scale_of(sv, s + 1) : 0.0f;
          u4_t w0, w1;
          pair_groups(q[s], q[s + 1], w0, w1);
          // reload the pair's slots with the groups PD positions ahead (the
          // next tile's first groups in the last cycle)
          const int tgt = gl + PD;
          const bool nxt = tgt >= np;
          const bool on = nxt && has_next;
          const int gg = nxt ? (has_next ? min(tgt - np, n - 1) : n - 1) : min(tgt, n - 1);
          q[s] = load_slot<LAY>(a, on ? cpn : cp, on ? cbn : cb, s, sb + gg);
          q[s + 1] = load_slot<LAY>(a, on ? cpn : cp, on ? cbn : cb, s + 1, sb + gg);
          __builtin_amdgcn_sched_barrier(0);
          const f4_t d0 = group_mfma<H>(xb, gl, w0);
#pragma unroll
          for (int r = 0; r < 4; ++r) accs[r] = fmaf(d0[r], sc0, accs[r]);
          const f4_t d1 = group_mfma<H>(xb, gl + 1, w1);
#pragma unroll
          for (int r = 0; r < 4; ++r) accs[r] = fmaf(d1[r], sc1, accs[r]);
        }
      } else {
#pragma unroll
        for (int s = 0; s < PD; ++s) {
          const int gl = fi + s;  // groups past n read the zeroed padding
          const float sc = (gl < n) ? scale_of(sv, s) : 0.0f;
          const f4_t d = group_mfma<H>(xb, gl, q[s]);
#pragma unroll
          for (int r = 0; r < 4; ++r) accs[r] = fmaf(d[r], sc, accs[r]);
          // reload this slot with the group PD positions ahead (the next
          // tile's first groups in the last cycle)
          const int tgt = gl + PD;
          const bool nxt = tgt >= np;
          const u4_t* cpl = (nxt && has_next) ? cpn : cp;
          const int gg = nxt ? (has_next ? min(tgt - np, n - 1) : n - 1) : min(tgt, n - 1);
          q[s] = load_codes<LAY>(cpl + code_off<LAY>(a, sb + gg));
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      sv = svn;
    }
    tile_outputs<TT>(a, v, r16, kq, w_cur, accs, fold, bv, bi, ro);
    v = vn;
    cp = cpn;
    cb = cbn;
    sp = spn;
    w_cur = w_next;
  }
}

// The tiles of one staged slice [sb, sb + n) of a run: the fp16 loop when
// the slice took the fp16 form (fold != 0), else the exact fallback.
template <int TT, int LAY>
__device__ __forceinline__ void run_slice(const GemvArgs& a, int64_t v0, int64_t v_end, int nwv,
                                          const unsigned char* xs, int r16, int kq, int trow, int sb, int n,
                                          const u4_t* cp, const u4_t* cb, const uint16_t* sp, u4_t (&q)[kRing],
                                          u4_t& sv, float fold, float (&bv)[4], int (&bi)[4], const RunOut& ro) {
  if (v0 >= v_end) return;  // uniform
  if constexpr (tries_f16<TT, true>()) {
    if (fold != 0.0f)
      run_tiles<TT, LAY, true>(a, v0, v_end, nwv, xs, r16, kq, trow, sb, n, cp, cb, sp, q, sv, fold, bv, bi, ro);
    else
      exact_run_tiles<TT, LAY>(a, v0, v_end, nwv, xs, r16, kq, trow, sb, n, bv, bi, ro);
  } else {
    run_tiles<TT, LAY, false>(a, v0, v_end, nwv, xs, r16, kq, trow, sb, n, cp, cb, sp, q, sv, kLevelScale, bv, bi, ro);
  }
}

// Run workgroup: a.run_tiles tiles per wave.  Workgroup b owns tiles
// [b*waves*nt, (b+1)*waves*nt); wave i streams tiles i, i + waves, ... of them,
// so the waves stay on adjacent tiles.  All of K is staged once (the planner
// guarantees it fits).  With a.fin_offset set the outputs are collected in
// LDS behind the staged activations and written when every wave is done.
// Built for one layout at a time (kLayTiled or kLayRow), eight scales per
// load.
template <int TT, int LAY>
__device__ __forceinline__ void run_workgroup(const GemvArgs& a, int64_t wg, unsigned char* smem) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nwv = blockDim.x >> 6;
  const int r16 = lane & 15, kq = lane >> 4;
  const int trow = min(r16, TT - 1);
  const int64_t tiles = (a.n_out + 15) / 16;
  const int64_t span = (int64_t)nwv * a.run_tiles;
  const int64_t v0 = wg * span + wave, v_end = min(tiles, (wg + 1) * span);
  unsigned char* xs = smem;
  const u4_t* cp = nullptr;
  const u4_t* cb = nullptr;
  const uint16_t* sp = nullptr;
  u4_t q[kRing];
  u4_t sv;
  // All of K staged at once (a.sk == a.G), or K in slices of a.sk groups
  // whose partial sums the LDS block carries from slice to slice.
  const bool sliced = a.sk < a.G;  // uniform
  // activations that fit kStageRegs chunks per thread are loaded first, then
  // the first tile's ring, then staged from the registers; larger ones are
  // staged after the ring is issued.  fold: the fp16 form's 2^-E, or 0
  const bool regs = !sliced && TT * a.G * (kGroup / 8) <= kStageRegs * (int)blockDim.x;  // uniform
  u4_t xr[kStageRegs];
  if (regs) prefetch_slice<TT>(a, 0, a.G, xr);
  float bv[4];
  int bi[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    bv[r] = __builtin_nanf("");
    bi[r] = -1;
  }
  float* const block = (a.fin_offset > 0 && (a.y || sliced)) ? reinterpret_cast<float*>(smem + a.fin_offset) : nullptr;
  float* const lane_out = block ? block + r16 * TT + 4 * kq : nullptr;
  float fold = 0.0f;
  if (regs) {  // all of K, staged from the registers (one pass below)
    if (v0 < v_end) {
      tile_ptr<LAY>(a, v0, r16, kq, cp, cb, sp);
      ring_prologue<LAY>(a, cp, cb, sp, 0, a.G, q, sv);
    }
    fold = stage_regs_shared<TT>(a, xs, 0, a.G, xr, tries_f16<TT, true>());
    __syncthreads();
  }
  // runs over K slices are built for the tiled layout only (the planner
  // slices no other; in the row-major kernels the loop's second pass cost
  // register spills)
  const int passes = LAY == kLayTiled ? (a.G + a.sk - 1) / a.sk : 1;
  for (int i = 0; i < passes; ++i) {  // uniform; one pass unless sliced
    const int sb = i * a.sk, n = min(a.G - sb, a.sk);
    if (!regs) {
      if (v0 < v_end) {
        tile_ptr<LAY>(a, v0, r16, kq, cp, cb, sp);
        ring_prologue<LAY>(a, cp, cb, sp, sb, n, q, sv);
      }
      if (sb > 0) __syncthreads();  // every wave is done with the previous slice
      fold = stage_slice<TT, true, tries_f16<TT, true>()>(a, xs, sb, sb + n);  // also waits for the ring's loads
    }
    run_slice<TT, LAY>(a, v0, v_end, nwv, xs, r16, kq, trow, sb, n, cp, cb, sp, q, sv, fold, bv, bi,
                       RunOut{lane_out, wg * span, sb == 0, sb + n == a.G});
  }
  if (block && a.y) {
    // every wave's tiles are in the block: write it to y token row by token
    // row (consecutive threads on consecutive outputs, whole lines), clipped
    // to n_out, with nontemporal stores at every row count (plain ones lose
    // the gain)
    __syncthreads();
    const int64_t row0 = wg * span * 16;  // < n_out: the grid holds no empty workgroup
    const int nr = (int)min(span * 16, a.n_out - row0);
    for (int t = 0; t < TT; ++t)
      for (int i = threadIdx.x; i < nr; i += (int)blockDim.x)
        __builtin_nontemporal_store(block[i * TT + t],
                                    (__attribute__((address_space(1))) float*)(a.y + (int64_t)t * a.n_out + row0 + i));
  }
  if (a.partial) {
    // per t: best of the lanes, of the waves, then of the workgroup
    int2* fin = reinterpret_cast<int2*>(smem);
    __syncthreads();  // the staging area is free now
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      // token row t lives in slot t % 4 of the lanes with kq = t / 4
      float val = bv[0];
      int id = bi[0];
#pragma unroll
      for (int r = 1; r < 4; ++r)
        if ((t & 3) == r) {
          val = bv[r];
          id = bi[r];
        }
      if (kq != (t >> 2)) id = -1;
      wave_argmax(val, id);
      if (lane == 0) fin[wave * TT + t] = int2{__float_as_int(val), id};
    }
    __syncthreads();
    if (wave == 0 && lane < TT) {
      float b = __builtin_nanf("");
      int i = -1;
      for (int w2 = 0; w2 < nwv; ++w2) {
        const int2 c = fin[w2 * TT + lane];
        if (better(__int_as_float(c.x), c.y, b, i)) {
          b = __int_as_float(c.x);
          i = c.y;
        }
      }
      st_partial(a.partial + wg * TT + lane, b, i);
    }
  }
}

template <int TT, int LAY>
__global__ void __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(4))) w4a16_run_kernel(GemvArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  run_workgroup<TT, LAY>(a, blockIdx.x, smem);
}

// Grouped launch of run workgroups: workgroup b runs workgroup b - wg_start of
// the last problem whose wg_start <= b; a problem planned without a run
// (its activations do not fit the LDS at once) runs a shared workgroup of one
// tile per wave instead.
template <int TT, int LAY>
__global__ void __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(4)))
w4a16_run_batch_kernel(const GemvArgs* __restrict__ table, int count) {
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
  if (a.run_tiles > 0)
    run_workgroup<TT, LAY>(a, b - a.wg_start, smem);
  else  // activations too large for one staging: whole-K slices, one tile per wave
    shared_workgroup<TT, 1, LAY>(a, b - a.wg_start, smem, true);
}

template <int TT, int RT, bool SHARED, int LAY>
__device__ __forceinline__ void tile_workgroup(const GemvArgs& a, int64_t wg, unsigned char* smem, bool grouped) {
  if constexpr (SHARED)
    shared_workgroup<TT, RT, LAY>(a, wg, smem, grouped);
  else
    split_workgroup<TT, RT, LAY>(a, wg, smem);
}

template <int TT, int RT, bool SHARED, int LAY>
__global__ void __launch_bounds__(SHARED && RT == 1 ? 1024 : 512)
    __attribute__((amdgpu_waves_per_eu(SHARED && RT == 1 ? 4 : 1))) w4a16_tile_kernel(GemvArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  tile_workgroup<TT, RT, SHARED, LAY>(a, blockIdx.x, smem, false);
}

// Grouped launch: workgroup b runs tile b - wg_start of the last problem whose
// wg_start <= b.
template <int TT, int RT, bool SHARED, int LAY>
__global__ void __launch_bounds__(SHARED && RT == 1 ? 1024 : 512)
    __attribute__((amdgpu_waves_per_eu(SHARED && RT == 1 ? 4 : 1)))
    w4a16_tile_batch_kernel(const GemvArgs* __restrict__ table, int count) {
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
  tile_workgroup<TT, RT, SHARED, LAY>(a, b - a.wg_start, smem, true);
}

// ------------------------------------------------------------- dispatch ----

// Above 64 KB of dynamic LDS a kernel has to opt in.  Each kernel function
// opts in once per device for the CU's whole LDS (the attribute is a
// property of the function on that device, so one call covers every later
// launch of it there); later launches check one bit.
template <typename F>
hipError_t allow_cu_lds(F* fn) {
  static std::atomic<unsigned long long> done{0};  // bit d: set on device d
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
  const unsigned long long bit = dev < 64 ? 1ull << dev : 0ull;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  const hipError_t e =
      hipFuncSetAttribute(reinterpret_cast<const void*>(fn), hipFuncAttributeMaxDynamicSharedMemorySize, kCuLds);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

template <int TT, int RT, bool SHARED, int LAY>
hipError_t launch_tiles(const GemvArgs& a, const GemvArgs* table, int count, const Plan& p, hipStream_t s) {
  const dim3 grid((unsigned)p.grid), block((unsigned)p.threads);
  if (p.lds > kLdsCap) {
    const hipError_t e = table ? allow_cu_lds(&w4a16_tile_batch_kernel<TT, RT, SHARED, LAY>)
                               : allow_cu_lds(&w4a16_tile_kernel<TT, RT, SHARED, LAY>);
    if (e != hipSuccess) return e;
  }
  if (table)
    hipLaunchKernelGGL((w4a16_tile_batch_kernel<TT, RT, SHARED, LAY>), grid, block, p.lds, s, table, count);
  else
    hipLaunchKernelGGL((w4a16_tile_kernel<TT, RT, SHARED, LAY>), grid, block, p.lds, s, a);
  return hipGetLastError();
}

template <int TT, bool SHARED>
hipError_t launch_rt(const GemvArgs& a, const GemvArgs* table, int count, const Plan& p, hipStream_t s) {
  if (p.tiled) {  // tiled-only kernels: one tile per wave, or two in split workgroups
    if (p.rt == 1) return launch_tiles<TT, 1, SHARED, kLayTiled>(a, table, count, p, s);
    if constexpr (!SHARED)
      if (p.rt == 2) return launch_tiles<TT, 2, false, kLayTiled>(a, table, count, p, s);
    return hipErrorInvalidValue;
  }
  if (p.rowmajor) {  // row-major-only kernels: paired whole-line loads
    switch (p.rt) {
      case 1: return launch_tiles<TT, 1, SHARED, kLayRow>(a, table, count, p, s);
      case 2: return launch_tiles<TT, 2, SHARED, kLayRow>(a, table, count, p, s);
      case 4: return launch_tiles<TT, 4, SHARED, kLayRow>(a, table, count, p, s);
      default: return hipErrorInvalidValue;
    }
  }
  switch (p.rt) {  // a grouped launch mixing both layouts
    case 1: return launch_tiles<TT, 1, SHARED, kLayAny>(a, table, count, p, s);
    case 2: return launch_tiles<TT, 2, SHARED, kLayAny>(a, table, count, p, s);
    case 4: return launch_tiles<TT, 4, SHARED, kLayAny>(a, table, count, p, s);
    default: return hipErrorInvalidValue;
  }
}

template <int TT, int LAY>
hipError_t launch_run(const GemvArgs& a, const GemvArgs* table, int count, const Plan& p, hipStream_t s) {
  const dim3 grid((unsigned)p.grid), block((unsigned)p.threads);
  if (p.lds > kLdsCap) {
    const hipError_t e =
        table ? allow_cu_lds(&w4a16_run_batch_kernel<TT, LAY>) : allow_cu_lds(&w4a16_run_kernel<TT, LAY>);
    if (e != hipSuccess) return e;
  }
  if (table)
    hipLaunchKernelGGL((w4a16_run_batch_kernel<TT, LAY>), grid, block, p.lds, s, table, count);
  else
    hipLaunchKernelGGL((w4a16_run_kernel<TT, LAY>), grid, block, p.lds, s, a);
  return hipGetLastError();
}

}  // namespace

// Launches the kernel of plan p for TT activation rows: one problem (a) or,
// with table set, a grouped launch over `count` problems.
template <int TT>
hipError_t launch_t(const GemvArgs& a, const GemvArgs* table, int count, const Plan& p, hipStream_t s) {
  if (p.variant == kRun)
    return p.tiled      ? launch_run<TT, kLayTiled>(a, table, count, p, s)
           : p.rowmajor ? launch_run<TT, kLayRow>(a, table, count, p, s)
                        : hipErrorInvalidValue;
  if (p.variant == kSplit) return launch_rt<TT, false>(a, table, count, p, s);
  if (p.variant == kShared) return launch_rt<TT, true>(a, table, count, p, s);
  if (table || p.variant != kDot || p.rt != 2) return hipErrorInvalidValue;
  if constexpr (TT <= kDotMaxT) {
    hipLaunchKernelGGL((w4a16_dot_kernel<TT, 2>), dim3((unsigned)p.grid), dim3((unsigned)p.threads), p.lds, s, a);
    return hipGetLastError();
  } else {
    return hipErrorInvalidValue;  // the planner never picks the dot kernel above kDotMaxT
  }
}

}  // namespace w4a16
