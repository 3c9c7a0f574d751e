// Planning, dispatch and the non-template kernels of libw4a16 (gfx950).
// The kernel templates live in w4a16_device.h; w4a16_kernels_tt.hip
// instantiates launch_t<TT> once per activation-row count.
#include <mutex>

#include "w4a16_device.h"

namespace w4a16 {

extern template hipError_t launch_t<1>(const GemvArgs&, const GemvArgs*, int, const Plan&, hipStream_t);
extern template hipError_t launch_t<2>(const GemvArgs&, const GemvArgs*, int, const Plan&, hipStream_t);
extern template hipError_t launch_t<3>(const GemvArgs&, const GemvArgs*, int, const Plan&, hipStream_t);
extern template hipError_t launch_t<4>(const GemvArgs&, const GemvArgs*, int, const Plan&, hipStream_t);
extern template hipError_t launch_t<5>(const GemvArgs&, const GemvArgs*, int, const Plan&, hipStream_t);
extern template hipError_t launch_t<6>(const GemvArgs&, const GemvArgs*, int, const Plan&, hipStream_t);
extern template hipError_t launch_t<7>(const GemvArgs&, const GemvArgs*, int, const Plan&, hipStream_t);
extern template hipError_t launch_t<8>(const GemvArgs&, const GemvArgs*, int, const Plan&, hipStream_t);
extern template hipError_t launch_t<9>(const GemvArgs&, const GemvArgs*, int, const Plan&, hipStream_t);
extern template hipError_t launch_t<10>(const GemvArgs&, const GemvArgs*, int, const Plan&, hipStream_t);
extern template hipError_t launch_t<11>(const GemvArgs&, const GemvArgs*, int, const Plan&, hipStream_t);
extern template hipError_t launch_t<12>(const GemvArgs&, const GemvArgs*, int, const Plan&, hipStream_t);
extern template hipError_t launch_t<13>(const GemvArgs&, const GemvArgs*, int, const Plan&, hipStream_t);
extern template hipError_t launch_t<14>(const GemvArgs&, const GemvArgs*, int, const Plan&, hipStream_t);
extern template hipError_t launch_t<15>(const GemvArgs&, const GemvArgs*, int, const Plan&, hipStream_t);
extern template hipError_t launch_t<16>(const GemvArgs&, const GemvArgs*, int, const Plan&, hipStream_t);

namespace {

constexpr unsigned short kBf16NaN = 0x7FC0;  // quiet NaN as a bf16 bit pattern

// ---------------------------------------------------------------- repack ----

// Row-major codes and scales -> tiled layout, one thread per 16 output bytes.
// Per tile the thread index runs over G * 64 code pieces (group g, row r,
// quarter q: bytes 64g + 16q .. of output row 16*tile + r) and then
// ceil(G/8) * 16 scale pieces (chunk c, row r: the bf16 scales of groups
// 8c .. 8c+7).  Output row o is input row row_ids[o] (o itself when row_ids
// is null).  Rows past N are written as zeros, as are groups past G; an
// output row whose id lies outside [0, n_rows) gets zero codes and NaN
// scales, so that its scores are NaN and never win an argmax (as a bad id
// of a gathered call gives).
__global__ void __launch_bounds__(256) w4a16_repack_kernel(const uint8_t* __restrict__ packed,
                                                           const uint16_t* __restrict__ scales,
                                                           const int32_t* __restrict__ row_ids, int64_t n_rows,
                                                           int64_t N, int K, uint8_t* __restrict__ tiled,
                                                           int64_t tile_bytes, int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int G = K / kGroup;
  const int chunks = (G + kTileChunkGroups - 1) / kTileChunkGroups;
  const int64_t per_tile = (int64_t)G * 64 + (int64_t)chunks * 16;
  const int64_t tile = i / per_tile;
  const int64_t rem = i - tile * per_tile;
  uint8_t* tb = tiled + tile * tile_bytes;
  u4_t v = {0u, 0u, 0u, 0u};
  if (rem < (int64_t)G * 64) {
    const int g = (int)(rem >> 6), r = (int)(rem >> 2) & 15, q = (int)rem & 3;
    const int64_t o = tile * 16 + r;
    const int64_t row = o >= N ? -1 : row_ids ? (int64_t)row_ids[o] : o;
    if (row >= 0 && row < n_rows) v = *reinterpret_cast<const u4_t*>(packed + row * (K / 2) + g * 64 + q * 16);
    *reinterpret_cast<u4_t*>(tb + (int64_t)(g >> 3) * kTileChunkBytes + (g & 7) * kTileGroupBytes + r * 64 +
                             q * 16) = v;
  } else {
    const int j = (int)(rem - (int64_t)G * 64);
    const int c = j >> 4, r = j & 15;
    const int64_t o = tile * 16 + r;
    const int64_t row = o >= N ? -1 : row_ids ? (int64_t)row_ids[o] : o;
    const bool ok = row >= 0 && row < n_rows;
    const bool bad_id = o < N && !ok;
    const int ng = min(kTileChunkGroups, G - c * kTileChunkGroups);
    unsigned short sc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      sc[e] = e >= ng ? 0 : ok ? scales[row * G + c * kTileChunkGroups + e] : bad_id ? kBf16NaN : 0;
    v = u4_t{sc[0] | ((unsigned)sc[1] << 16), sc[2] | ((unsigned)sc[3] << 16), sc[4] | ((unsigned)sc[5] << 16),
             sc[6] | ((unsigned)sc[7] << 16)};
    *reinterpret_cast<u4_t*>(tb + (int64_t)c * kTileChunkBytes + ng * kTileGroupBytes + r * 16) = v;
  }
}

// ---------------------------------------------------------- argmax final ----

// Workgroup t reduces the nparts partials of token row t: each of its 256
// threads loads up to kArgmaxBatch of them at once (one memory round trip
// per 2,048 partials; the dot variant's 15,520 partials of the lm_head took
// 15 us less than with one load at a time), then the waves and the
// workgroup reduce.  The rule (larger value, then lower id; id -1 never
// wins) is a total order, so the result does not depend on the order of
// the reduction.
constexpr int kArgmaxThreads = 256, kArgmaxBatch = 8;

__global__ void __launch_bounds__(kArgmaxThreads) w4a16_argmax_final(const int2* partial, int64_t nparts, int T,
                                                                     int32_t* id_out, float* val_out) {
  __shared__ float sv[kArgmaxThreads / 64];
  __shared__ int si[kArgmaxThreads / 64];
  const int t = blockIdx.x;
  float bv = __builtin_nanf("");
  int bi = -1;
  for (int64_t j0 = threadIdx.x; j0 < nparts; j0 += (int64_t)kArgmaxThreads * kArgmaxBatch) {
    int2 p[kArgmaxBatch];
#pragma unroll
    for (int u = 0; u < kArgmaxBatch; ++u) {
      const int64_t j = j0 + (int64_t)u * kArgmaxThreads;
      p[u] = j < nparts ? partial[j * T + t] : int2{0, -1};
    }
#pragma unroll
    for (int u = 0; u < kArgmaxBatch; ++u) {
      const float v = __int_as_float(p[u].x);
      if (better(v, p[u].y, bv, bi)) {
        bv = v;
        bi = p[u].y;
      }
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
    for (int w = 1; w < kArgmaxThreads / 64; ++w)
      if (better(sv[w], si[w], bv, bi)) {
        bv = sv[w];
        bi = si[w];
      }
    if (id_out) id_out[t] = bi;
    if (val_out) val_out[t] = bi < 0 ? __builtin_nanf("") : bv;
  }
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
    case 9: return f(std::integral_constant<int, 9>{});
    case 10: return f(std::integral_constant<int, 10>{});
    case 11: return f(std::integral_constant<int, 11>{});
    case 12: return f(std::integral_constant<int, 12>{});
    case 13: return f(std::integral_constant<int, 13>{});
    case 14: return f(std::integral_constant<int, 14>{});
    case 15: return f(std::integral_constant<int, 15>{});
    case 16: return f(std::integral_constant<int, 16>{});
    default: return hipErrorInvalidValue;
  }
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Groups rounded up to whole cycles of the load ring (the staged rows hold
// the ring's padded slots too).
int ring_groups(int g) { return (int)(cdiv(g, kRing) * kRing); }

}  // namespace

bool parse_tile(const char* text, Tile* t) {
  char kind[16] = {0};
  int rt = 0, nw = 0;
  if (!text || std::sscanf(text, "%15[a-z],%d,%d", kind, &rt, &nw) != 3) return false;
  if (std::strcmp(kind, "run") == 0) {
    if (rt < 1 || rt > 16 || nw < 1 || nw > 16) return false;
    *t = Tile{kRun, rt, nw};
    return true;
  }
  const bool split = std::strcmp(kind, "split") == 0, shared = std::strcmp(kind, "shared") == 0;
  if (!(split || shared) || !(rt == 1 || rt == 2 || rt == 4) || nw < 1) return false;
  if (nw > (shared && rt == 1 ? 16 : 8)) return false;
  *t = Tile{split ? kSplit : kShared, rt, nw};
  return true;
}

// Split tiling: rt 16-row tiles per workgroup; K is cut into per-wave ranges
// of gpw groups (a multiple of the 8-group ring, so that 8-scale vector loads
// stay aligned; the last wave may hold fewer) over at most nw_max waves.  A
// wave's LDS area holds its staged activation slice of sk groups (the whole
// range when half a CU's LDS allows it, else a multiple of 8; swizzled
// chunks, no padding between token rows) and later its partial sums; the
// final values overwrite wave 0's partials in place.  At most half a CU, so
// that two workgroups share a CU (the split kernels are built for at most
// eight waves).
static void plan_split(GemvArgs& a, int T, int rt, int nw_max, Plan* p) {
  const int cap = kCuLds / 2;
  for (int nw = std::max(1, std::min(nw_max, a.G));; --nw) {
    const int gpw = (int)(cdiv(cdiv(a.G, nw), kRing) * kRing);
    const int nw_eff = (int)cdiv(a.G, gpw);
    const int per_wave = (cap / nw_eff) & ~15;
    int sk = per_wave / (2 * T) / kGroup;
    if (sk >= gpw)
      sk = std::min(gpw, a.G);
    else if (sk >= kRing)
      sk -= sk % kRing;
    else if (nw > 1)
      continue;
    else
      sk = kRing;  // unreachable for T <= 16: one wave always fits 20 groups
    a.nw = nw_eff;
    a.gpw = gpw;
    a.sk = sk;
    a.xs_stride = ring_groups(sk) * kGroup;
    const int wave_lds = std::max(T * a.xs_stride * 2, rt * T * 16 * 4);
    a.wave_lds = (wave_lds + 15) & ~15;
    a.fin_offset = 0;
    p->lds = nw_eff * a.wave_lds;
    if (p->lds > cap && nw > 1) continue;
    p->threads = nw_eff * 64;
    p->grid = cdiv(a.n_out, 16LL * rt);
    return;
  }
}

// LDS of a workgroup that stages activations for all its waves: up to eight
// waves it may take half a CU (two such workgroups per CU), above that all
// of it.
static int shared_cap(int nwv) { return nwv > 8 ? kCuLds : kCuLds / 2; }

// Shared tiling: nwv waves of rt 16-row tiles per workgroup over all of K; the
// activation slice staged in LDS holds sk groups (all of K when the LDS
// allows it, else a multiple of the 8-group ring) of every token row, and
// nothing else: the staging's flag words, the slice maxima and the argmax
// partials of the waves reuse the staging area.
static void plan_shared(GemvArgs& a, int T, int rt, int nwv, Plan* p) {
  const int sk_cap = shared_cap(nwv) / (T * kGroup * 2);
  const int sk = ring_groups(a.G) <= sk_cap ? a.G : std::max(kRing, sk_cap - sk_cap % kRing);
  a.nw = nwv;
  a.gpw = a.G;
  a.sk = sk;
  a.xs_stride = ring_groups(sk) * kGroup;
  a.wave_lds = 0;
  a.fin_offset = 0;
  p->lds = std::max(T * a.xs_stride * 2, nwv * T * 8);
  p->threads = nwv * 64;
  p->grid = cdiv(a.n_out, 16LL * nwv * rt);
}

// Run tiling: nwv waves of nt whole tiles each, eight scales per load, all
// of K staged at once (shared_cap); returns false otherwise.  On the tiled
// layout, when all of K fits but leaves no room for the output block below,
// K goes in slices of sk groups (a multiple of the ring) and the partial
// sums stay in the block from slice to slice (27B-class body pass at T = 13
// and 16: +5 points against whole-K runs storing per tile).  Activations
// that do not fit at all are not sliced into runs: the down projection
// (K = 17,408) lost 4-5 points at T = 3-12 that way against the shared
// workgroups a grouped launch runs for it.
//
// When the LDS share still holds them behind the staged activations, the
// workgroup's T x 16*nt*nwv outputs are collected there and written at its
// end as whole rows of nontemporal stores (fin_offset: their offset).
// Output stores are far dearer than their share of the bytes in the middle
// of the weight stream: timing-only copies of the body pass that drop them
// run 3.7, 7 and 8 points of 8 TB/s faster at T = 4, 8 and 16, and one that
// writes a quarter of them at T = 4 is as fast as none.  Collected, the
// pass gains 1-2 points at T = 3-8 and about 4 at T = 9-10.
static bool plan_run(GemvArgs& a, int T, int nt, int nwv, Plan* p) {
  if (!a.vec_scales) return false;
  const int64_t cap = shared_cap(nwv);
  const int64_t row_bytes = (int64_t)T * kGroup * 2;          // one staged group of every token row
  const int64_t out_bytes = (int64_t)T * nwv * nt * 16 * 4;  // fp32 outputs of the workgroup's rows
  const int64_t whole = ring_groups(a.G) * row_bytes;
  int sk = a.G;
  bool collect = whole + out_bytes <= cap;
  if (!collect) {
    const int slice = cap > out_bytes ? (int)((cap - out_bytes) / row_bytes) / kRing * kRing : 0;
    if (a.tiled && kSlicedRuns && whole <= cap && slice >= kRing && slice < a.G) {
      sk = slice;
      collect = true;
    } else if (whole > cap) {
      return false;
    }
  }
  a.nw = nwv;
  a.gpw = a.G;
  a.sk = sk;
  a.xs_stride = ring_groups(sk) * kGroup;
  a.wave_lds = 0;
  a.run_tiles = nt;
  const int64_t xs_bytes = ring_groups(sk) * row_bytes;  // a multiple of 16
  a.fin_offset = collect ? (int)xs_bytes : 0;
  p->lds = std::max((int)(collect ? xs_bytes + out_bytes : xs_bytes), nwv * T * 8);
  p->threads = nwv * 64;
  p->grid = cdiv(cdiv(a.n_out, 16), (int64_t)nwv * nt);
  return true;
}

Plan plan_tile(GemvArgs& a, int T, const Tile& t, bool tiled_kernel, bool row_kernel, bool batch) {
  Plan p{};
  p.variant = t.shape;
  p.rowmajor = row_kernel && !tiled_kernel;
  // the tiled-layout kernels stream one tile per wave (two in split workgroups)
  p.rt = tiled_kernel && !(t.shape == kSplit && t.rt == 2) ? 1 : t.rt;
  p.tiled = tiled_kernel;
  a.vec_scales = (a.tiled || (a.G % 8 == 0 && (reinterpret_cast<uintptr_t>(a.scales) & 15) == 0)) ? 1 : 0;
  if (t.shape == kRun) {
    // runs are built for one layout at a time: a grouped launch mixing the
    // layouts takes shared workgroups of one tile per wave instead
    const bool one_layout = tiled_kernel || p.rowmajor;
    p.rt = 1;
    if (one_layout && plan_run(a, T, t.rt, t.nw, &p)) return p;
    // The activations do not fit: a shared workgroup of one tile per wave
    // stages K in slices.  A grouped launch keeps the run kernel (which
    // runs such problems this way, run_tiles = 0); a single launch switches.
    a.run_tiles = 0;
    plan_shared(a, T, 1, t.nw, &p);
    p.variant = batch && one_layout ? kRun : kShared;
    return p;
  }
  if (t.shape == kShared)
    plan_shared(a, T, p.rt, t.nw, &p);
  else
    plan_split(a, T, p.rt, t.nw, &p);
  return p;
}

// The measurement overrides of the tile choice: one for single launches,
// one for grouped launches, each packed into one word (0: none) so that
// plans read them without a lock.  Set from W4A16_TILE / W4A16_BATCH_TILE
// once per process, and by set_tile_override (w4a16_set_tile).
namespace {
uint32_t pack_tile(const Tile& t) { return 1u | (uint32_t)t.shape << 1 | (uint32_t)t.rt << 4 | (uint32_t)t.nw << 10; }
Tile unpack_tile(uint32_t w) { return Tile{(int)(w >> 1 & 7), (int)(w >> 4 & 63), (int)(w >> 10 & 63)}; }
std::atomic<uint32_t> g_tile_override[2];
std::once_flag g_tile_env_once;
void read_tile_env() {
  Tile t;
  if (parse_tile(std::getenv("W4A16_TILE"), &t)) g_tile_override[0].store(pack_tile(t));
  if (parse_tile(std::getenv("W4A16_BATCH_TILE"), &t)) g_tile_override[1].store(pack_tile(t));
}
}  // namespace

bool tile_override(bool batch, Tile* t) {
  std::call_once(g_tile_env_once, read_tile_env);
  const uint32_t w = g_tile_override[batch ? 1 : 0].load(std::memory_order_relaxed);
  if (!w) return false;
  *t = unpack_tile(w);
  return true;
}

bool set_tile_override(bool batch, const char* spec) {
  std::call_once(g_tile_env_once, read_tile_env);
  if (!spec || !*spec) {
    g_tile_override[batch ? 1 : 0].store(0);
    return true;
  }
  Tile t;
  if (!parse_tile(spec, &t)) return false;
  g_tile_override[batch ? 1 : 0].store(pack_tile(t));
  return true;
}

// (A grouped decode pass at T = 2: 8 waves 82.7 % of 8 TB/s against 71.8 %
// for 4, whose LDS share keeps the 17,408-column problems to 8 waves a CU;
// at T = 1 both give 84-86 %.)
int shared_waves(int T, int64_t K) {
  if ((int64_t)T * ring_groups((int)(K / kGroup)) * kGroup * 2 > shared_cap(8)) return 16;
  return T <= 1 ? 4 : 8;
}

// Default matrix-core tiling of a single launch (cus: compute units of the
// device), from the MI355X sweeps over the workload shapes and a grid of
// others (N 512 - 131,072, K 1,024 - 17,408, T 1 - 16, both layouts):
//   - tiled, >= 4,096 tiles: runs of 4 tiles x 16 waves when one round of
//     them fills the CUs (the vocabulary head), else 2 tiles x 8 waves; where
//     the staging is dear (below), one round of 16-wave runs of as many tiles
//     per wave as that takes, while it keeps three quarters of the CUs busy;
//   - row-major, >= 4,096 tiles: shared workgroups of 8 waves x 2 tiles;
//   - 1,024 - 4,095 tiles: shared workgroups of one tile per wave, 4 waves
//     (8 where that makes one full round); where the staging is dear, one
//     round of 4, 8 or 16 waves;
//   - shorter matrices, T <= 8: from T = 2 and three quarters of a round,
//     4-wave shared workgroups too; else split workgroups that cut K over
//     their waves to put ~12 waves of weight loads on every CU, two tiles
//     per workgroup from 1.25 tiles per CU;
//   - shorter matrices, T > 8: shared workgroups of 4 waves (a split wave's
//     staged slice would hold too few groups).
// W4A16_TILE = "split|shared|run,rt,waves" overrides the choice (for
// measurement).
Plan plan_mfma(GemvArgs& a, int T, int cus) {
  const int64_t tiles = cdiv(a.n_out, 16);
  Tile t;
  const int64_t ncu = std::max(cus, 1);
  // Where the staging is dear (tiled from T = 5, row-major from T = 8, and
  // wherever T rows of K do not fit half a CU's LDS, so that smaller
  // workgroups would stage in slices), one round of workgroups, one per CU,
  // each staging the activations once for as many tiles as the CU's share:
  // the fewest waves (4, 8, 16) whose workgroups fit one round, then runs of
  // several tiles per wave.  (Mid-size shapes at T = 8: 16,384 x 5,120
  // tiled 16.7 us against 24.7 for 16-wave workgroups, row-major 21 against
  // 37; at T = 4, 32,768 x 17,408 tiled 54 against 65.)
  const bool dear = (a.tiled ? T > 4 : T >= 8) || (int64_t)T * ring_groups(a.G) * kGroup * 2 > shared_cap(8);
  if (tiles >= 4096 && a.tiled) {
    if (dear) {  // 6,250 tiles: 2 per wave; the vocabulary head: 4
      const int rt = (int)std::min<int64_t>(16, cdiv(tiles, 16 * ncu));
      // a round that would leave a quarter of the CUs idle: 8-wave runs of 2
      t = cdiv(tiles, 16LL * rt) * 4 >= 3 * ncu ? Tile{kRun, rt, 16} : Tile{kRun, 2, 8};
    } else {
      // one round of 16-wave runs of 4 tiles when it fills nine tenths of the
      // CUs (the vocabulary head: 243 workgroups), else 8-wave runs of 2
      // tiles, two workgroups per CU (65,536 x 5,120: 32 us against 73 us for
      // the 64 workgroups of 4 x 16; 131,072 rows: 58 against 89)
      t = cdiv(tiles, 64) * 10 >= 9 * ncu ? Tile{kRun, 4, 16} : Tile{kRun, 2, 8};
    }
  } else if (T == 1 && tiles >= 1024 && tiles < 4096 && !a.partial && !a.row_ids)
    t = Tile{kSplit, 1, 4};  // a plain matmul (34,816 x 5,120: 20.3 us against 23.8 for shared workgroups of 4 waves)
  else if (tiles >= 4096)  // row-major: 248,320 x 5,120 with argmax, 114.5 us against 118.9 for 4 x 8 at T = 1
    t = Tile{kShared, 2, 8};
  else if (tiles >= 1024 && dear)
    t = Tile{kShared, 1, cdiv(tiles, 4) <= ncu ? 4 : cdiv(tiles, 8) <= ncu ? 8 : 16};
  else if (tiles >= 1024 && T <= 8 && cdiv(tiles, 8) <= ncu && cdiv(tiles, 8) * 10 >= 9 * ncu)
    t = Tile{kShared, 1, 8};  // one full round of 8-wave workgroups (the 32,768-row draft head: 256)
  else if (tiles >= 1024 || T > 8)  // above 8 rows a split wave stages too little K per slice
    t = Tile{kShared, 1, 4};
  else if (T >= 2 && tiles >= 3 * ncu)  // still three quarters of a round of 4-wave workgroups,
    t = Tile{kShared, 1, 4};             // each staging once for 4 tiles (12,288 x 5,120 at T = 8: 16 us vs 23)
  else if (4 * tiles >= 5 * ncu)
    // Up to 64 groups of K, 8-wave split workgroups of one tile, each wave
    // staging and streaming 8 groups (5,120 x 5,120 tiled at T = 1: 7.6 us
    // against 8.0 for 2 tiles per workgroup; 9.0 against 9.9 at T = 4).
    // Longer K: at T = 1 four waves of one tile (5,120 x 17,408: 15.4 us
    // against 16.8), above it split workgroups of 2 tiles (row-major 44 us
    // against 65 for shared workgroups at T = 8; tiled 25 against 27 at T = 4)
    t = a.G <= 64 ? Tile{kSplit, 1, 8} : T == 1 ? Tile{kSplit, 1, 4} : Tile{kSplit, 2, 8};
  else
    t = Tile{kSplit, 1, (int)std::min<int64_t>(8, std::max<int64_t>(1, cdiv(12LL * std::max(cus, 1), tiles)))};
  tile_override(false, &t);
  return plan_tile(a, T, t, a.tiled != 0, a.tiled == 0, false);
}

// Tiling of the dot variant: 2 rows per wave (32 lanes per row), 8 waves,
// activations staged per workgroup in slices of at most 8 chunks per lane
// (64 groups), each staged row a whole number of 4-group blocks (the
// staging fills 64 chunk positions per copy); the final values reuse the
// staging area.
Plan plan_dot(GemvArgs& a, int T) {
  Plan p{};
  p.variant = kDot;
  p.rt = 2;  // rows per wave
  const int nw = 8;
  p.threads = nw * 64;
  const int L = 64 / p.rt;
  p.grid = cdiv(a.n_out, (int64_t)p.rt * nw);
  const int max_sk_regs = 8 * L / 4;                   // CPL chunks per lane, 4 chunks per group
  const int sk_lds = (kLdsCap / (T * kGroup * 2)) & ~3;  // whole 4-group blocks per row
  a.nw = nw;
  a.sk = std::max(1, std::min({a.G, max_sk_regs, sk_lds}));
  a.gpw = a.G;
  a.xs_stride = (int)cdiv(a.sk, 4) * 4 * kGroup;
  a.wave_lds = 0;
  a.fin_offset = 0;
  const int fin_bytes = (int)cdiv(nw * p.rt, 16) * T * 16 * 4;
  p.lds = std::max(T * a.xs_stride * 2, fin_bytes);
  return p;
}

namespace {

// Measurement: every 16-byte word of src read once, four nontemporal loads
// in flight per thread, workgroup b over the b-th contiguous share.  The
// words are folded by XOR into one value per thread, stored to sink, so that
// no load can be dropped.
__global__ void __launch_bounds__(256) w4a16_stream_read_kernel(const u4_t* __restrict__ src, int64_t n16,
                                                                unsigned* __restrict__ sink) {
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t b = (int64_t)blockIdx.x * per, e = min(n16, b + per);
  unsigned acc = 0;
  int64_t i = b + threadIdx.x;
  for (; i + 3 * 256 < e; i += 4 * 256) {
    const u4_t v0 = ld_global_nt(src + i), v1 = ld_global_nt(src + i + 256);
    const u4_t v2 = ld_global_nt(src + i + 512), v3 = ld_global_nt(src + i + 768);
    acc ^= (v0.x ^ v0.y ^ v0.z ^ v0.w) ^ (v1.x ^ v1.y ^ v1.z ^ v1.w) ^ (v2.x ^ v2.y ^ v2.z ^ v2.w) ^
           (v3.x ^ v3.y ^ v3.z ^ v3.w);
  }
  for (; i < e; i += 256) {
    const u4_t v = ld_global_nt(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  st_global(sink + (int64_t)blockIdx.x * 256 + threadIdx.x, acc);
}

}  // namespace

hipError_t launch_stream_read(const void* src, int64_t bytes, unsigned* sink, int workgroups, hipStream_t s) {
  hipLaunchKernelGGL(w4a16_stream_read_kernel, dim3((unsigned)workgroups), dim3(256), 0, s,
                     static_cast<const u4_t*>(src), bytes / 16, sink);
  return hipGetLastError();
}

int64_t max_workgroups(int64_t n_out) { return cdiv(n_out, 16); }

hipError_t launch(const GemvArgs& a, const Plan& p, int T, hipStream_t s) {
  return for_t(T, [&](auto tt) { return launch_t<decltype(tt)::value>(a, nullptr, 0, p, s); });
}

hipError_t launch_batch(const GemvArgs* table_dev, int count, const Plan& p, int T, hipStream_t s) {
  GemvArgs unused{};
  return for_t(T, [&](auto tt) { return launch_t<decltype(tt)::value>(unused, table_dev, count, p, s); });
}

hipError_t launch_repack(const uint8_t* packed, const uint16_t* scales, const int32_t* row_ids, int64_t n_rows,
                         int64_t N, int32_t K, uint8_t* tiled, hipStream_t s) {
  const int G = K / kGroup;
  const int64_t tiles = cdiv(N, 16);
  const int64_t total = tiles * ((int64_t)G * 64 + cdiv(G, kTileChunkGroups) * 16);
  hipLaunchKernelGGL(w4a16_repack_kernel, dim3((unsigned)cdiv(total, 256)), dim3(256), 0, s, packed, scales, row_ids,
                     n_rows, N, K, tiled, tiled_tile_bytes(G), total);
  return hipGetLastError();
}

hipError_t launch_argmax_final(const int2* partial, int64_t nparts, int T, int32_t* id, float* val, hipStream_t s) {
  hipLaunchKernelGGL(w4a16_argmax_final, dim3((unsigned)T), dim3(kArgmaxThreads), 0, s, partial, nparts, T, id, val);
  return hipGetLastError();
}

}  // namespace w4a16
