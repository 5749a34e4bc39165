// Force pass: LDS-tiled all-pairs softened gravity for gfx950.
//
// Decomposition (the tiled scheme of "Cuda Nbody Notes" and of section 3.1
// of the "CUDA N-Body Simulation" README, rebuilt for 64-wide wavefronts):
//  - each lane keeps K i-bodies and their accumulators in VGPRs;
//  - a block of `waves` wavefronts stages j-bodies in LDS tiles of T bodies;
//    every lane of a wave reads the same LDS address, which the LDS serves as
//    a broadcast (the CUDA Handbook's shared-memory page makes the same point
//    for warps);
//  - a wave may be split into lane groups that take interleaved j-bodies of
//    each tile (two LDS addresses per read instead of one), so K i-bodies
//    per lane need fewer i-bodies per block and small n still fills the chip;
//  - the block may split j over S parts (waves / S waves per part): each part
//    walks its own contiguous range of tiles and the part sums are added in
//    ascending part order through LDS at the end.  This keeps small n
//    occupying the chip without a global workspace or atomics;
//  - tiles are double-buffered: the next tile's global loads are issued
//    before the current tile's arithmetic and written to the other LDS buffer
//    after it, so there is one barrier per tile;
//  - the i side may be a sub-range [i0, i0 + ni) of the bodies (one GPU's
//    share when the pass is split by i); output row r is body i0 + r;
//  - ragged n: staged indices are clamped into [0, n) and the mass of every
//    padding slot is zeroed, so the inner loop has no bounds test and a
//    padding term adds exactly +0 (README section 3.1 guards the same tail
//    with a loop bound instead).
// No MFMA: the pair step is a reciprocal square root and a handful of
// multiply-adds per pair, not a dense contraction.
#include "nbody_common.hpp"
#include "nbody_internal.hpp"

namespace nbody {

// OCC > 0 asks the compiler to fit OCC waves per SIMD (it then caps VGPRs at
// 512 / OCC); 0 leaves the register budget to the compiler.
//
// POT = true also sums phi_i = sum_{j != i} m_j (r^2 + eps^2)^{-1/2}
// (two-level like the acceleration; the j = i pair is dropped by an index
// test, three more VALU ops per pair) and stores Phi_i = -G phi_i in the
// output's w.
//
// LG > 1 splits each wave into LG lane groups of 64 / LG lanes: lane group g
// takes the tile's bodies jj with jj % LG == g (LG consecutive float4s per LDS
// read, so the groups hit different banks), and a wave covers 64 / LG columns
// of K i-bodies.  A wave then holds K i-bodies per lane with LG times fewer
// i-bodies per block, which keeps small n filling the chip with K > 1.  The
// groups' sums are added in ascending g (ds_bpermute) once, after the last
// tile, before the parts are added.
//
// block0 is the number of the launch's first block: a grid too large for one
// launch goes out as several, and block b of the grid computes the same rows
// in any of them.
template <int K, int T, int WAVES, int S, int U, int OCC, class L, bool POT = false, int LG = 1>
__global__ __launch_bounds__(WAVES *kWave)
__attribute__((amdgpu_waves_per_eu(OCC > 0 ? OCC : 1))) void force_tile_kernel(
    L lay, int n, int i0, int ni, int n_tiles, int tiles_per_part, float G, float eps2,
    int block0) {
  constexpr int GW = WAVES / S;            // i-groups (waves) per part
  constexpr int CW = kWave / LG;           // i columns per wave
  constexpr int NTHREADS = WAVES * kWave;  // threads per block
  constexpr int LOADS = (S * T) / NTHREADS;
  static_assert(WAVES % S == 0, "waves must be a multiple of the split");
  static_assert((S * T) % NTHREADS == 0, "staged bodies must divide evenly over threads");
  static_assert(kWave % LG == 0 && T % LG == 0, "lane groups must divide the wave and the tile");
  static_assert(S == 1 || GW * K * (POT ? 4 : 3) * kWave <= 2 * S * T * 4,
                "one part's sums must fit in the tile buffers");
  __shared__ float4 tile[2][S * T];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int col = lane % CW;
  const int lg = lane / CW;
  const int part = wave / GW;
  const int grp = wave % GW;
  const int base = (block0 + (int)blockIdx.x) * (GW * CW * K) + grp * CW + col;

  float xi[K], yi[K], zi[K], ax[K], ay[K], az[K], ap[K];
#pragma unroll
  for (int q = 0; q < K; ++q) {
    const int i = base + q * GW * CW;
    const float4 b = lay.load(i0 + (i < ni ? i : ni - 1));
    xi[q] = b.x;
    yi[q] = b.y;
    zi[q] = b.z;
    ax[q] = 0.0f;
    ay[q] = 0.0f;
    az[q] = 0.0f;
    ap[q] = 0.0f;
  }

  // Staging slot e of a step holds body jj = e % T of part e / T's tile.
  // The padding test is kept apart from the load and applied in stash(), so
  // the global load stays in flight across the current tile's arithmetic.
  float4 reg[LOADS];
  bool real[LOADS];
  auto fetch = [&](int step) {
#pragma unroll
    for (int r = 0; r < LOADS; ++r) {
      const int e = tid + r * NTHREADS;
      const int j = ((e / T) * tiles_per_part + step) * T + (e % T);
      reg[r] = lay.load(j < n ? j : n - 1);
      real[r] = j < n;
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int r = 0; r < LOADS; ++r) {
      float4 b = reg[r];
      b.w = real[r] ? b.w : 0.0f;
      tile[buf][tid + r * NTHREADS] = b;
    }
  };

  fetch(0);
  stash(0);
  for (int step = 0; step < tiles_per_part; ++step) {
    __syncthreads();
    const int cur = step & 1;
    const bool more = step + 1 < tiles_per_part;
    if (more) fetch(step + 1);
    if (part * tiles_per_part + step < n_tiles) {
      const float4 *tp = &tile[cur][part * T];
      const int j0 = (part * tiles_per_part + step) * T;
      float px[K], py[K], pz[K], pp[K];
#pragma unroll
      for (int q = 0; q < K; ++q) {
        px[q] = 0.0f;
        py[q] = 0.0f;
        pz[q] = 0.0f;
        pp[q] = 0.0f;
      }
#pragma unroll U
      for (int jj = 0; jj < T / LG; ++jj) {
        const float4 b = tp[jj * LG + lg];
#pragma unroll
        for (int q = 0; q < K; ++q) {
          if constexpr (POT) {
            const float mp = (j0 + jj * LG + lg == i0 + base + q * GW * CW) ? 0.0f : b.w;
            pair_accel_pot(b.x, b.y, b.z, b.w, mp, xi[q], yi[q], zi[q], eps2, px[q], py[q],
                           pz[q], pp[q]);
          }
          else
            pair_accel(b.x, b.y, b.z, b.w, xi[q], yi[q], zi[q], eps2, px[q], py[q], pz[q]);
        }
      }
#pragma unroll
      for (int q = 0; q < K; ++q) {
        ax[q] += px[q];
        ay[q] += py[q];
        az[q] += pz[q];
        if constexpr (POT) ap[q] += pp[q];
      }
    }
    if (more) stash(cur ^ 1);
  }

  if constexpr (LG > 1) {
    // lane group 0 adds groups 1 .. LG-1 in ascending order; the other
    // groups' lanes carry unused values from here on
#pragma unroll
    for (int q = 0; q < K; ++q) {
      float sx = ax[q], sy = ay[q], sz = az[q], sp = ap[q];
#pragma unroll
      for (int g = 1; g < LG; ++g) {
        sx += __shfl(ax[q], col + g * CW);
        sy += __shfl(ay[q], col + g * CW);
        sz += __shfl(az[q], col + g * CW);
        if constexpr (POT) sp += __shfl(ap[q], col + g * CW);
      }
      ax[q] = sx;
      ay[q] = sy;
      az[q] = sz;
      ap[q] = sp;
    }
  }

  if constexpr (S > 1) {
    float *red = reinterpret_cast<float *>(&tile[0][0]);
    constexpr int NC = POT ? 4 : 3;  // sums per body
    if constexpr ((S - 1) * GW * K * NC * kWave <= 2 * S * T * 4) {
      // All parts p >= 1 write their sums into the (now idle) tile buffers at
      // once; after one barrier part 0 adds them in ascending p.
      __syncthreads();
      if (part > 0) {
#pragma unroll
        for (int q = 0; q < K; ++q) {
          const int o = (((part - 1) * GW + grp) * K + q) * NC * kWave + lane;
          red[o] = ax[q];
          red[o + kWave] = ay[q];
          red[o + 2 * kWave] = az[q];
          if constexpr (POT) red[o + 3 * kWave] = ap[q];
        }
      }
      __syncthreads();
      if (part == 0) {
        for (int p = 1; p < S; ++p) {
#pragma unroll
          for (int q = 0; q < K; ++q) {
            const int o = (((p - 1) * GW + grp) * K + q) * NC * kWave + lane;
            ax[q] += red[o];
            ay[q] += red[o + kWave];
            az[q] += red[o + 2 * kWave];
            if constexpr (POT) ap[q] += red[o + 3 * kWave];
          }
        }
      }
    } else {
      // Part p's sums go through the tile buffers one part at a time and
      // part 0 adds them in ascending p.
      for (int p = 1; p < S; ++p) {
        __syncthreads();
        if (part == p) {
#pragma unroll
          for (int q = 0; q < K; ++q) {
            const int o = ((grp * K + q) * NC) * kWave + lane;
            red[o] = ax[q];
            red[o + kWave] = ay[q];
            red[o + 2 * kWave] = az[q];
            if constexpr (POT) red[o + 3 * kWave] = ap[q];
          }
        }
        __syncthreads();
        if (part == 0) {
#pragma unroll
          for (int q = 0; q < K; ++q) {
            const int o = ((grp * K + q) * NC) * kWave + lane;
            ax[q] += red[o];
            ay[q] += red[o + kWave];
            az[q] += red[o + 2 * kWave];
            if constexpr (POT) ap[q] += red[o + 3 * kWave];
          }
        }
      }
    }
  }

  if (part == 0 && lg == 0) {
#pragma unroll
    for (int q = 0; q < K; ++q) {
      const int i = base + q * GW * CW;
      if constexpr (POT) {
        if (i < ni) lay.store4(i, G * ax[q], G * ay[q], G * az[q], -G * ap[q]);
      } else {
        if (i < ni) lay.store(i, G * ax[q], G * ay[q], G * az[q]);
      }
    }
  }
}

// LDS-free variant (an ablation of the staging choice): each wave reads the
// j-bodies straight from memory, in ascending j, with the same two-level sum
// over chunks of T.  MODE 0 lets the compiler turn the wave-uniform loads into
// scalar (SGPR) loads; MODE 1 forces vector loads of one address per wave
// (the cache-only scheme the Handbook page mentions).  The j loop stops at
// n (a wave-uniform bound), so there is no padding; with S = 1 and the same T
// the sums are bitwise equal to the LDS kernel's.
template <int K, int T, int WAVES, int MODE, int OCC>
__global__ __launch_bounds__(WAVES *kWave)
__attribute__((amdgpu_waves_per_eu(OCC > 0 ? OCC : 1))) void force_stream_kernel(
    const float4 *__restrict__ pm, int n, int i0, int ni, float G, float eps2,
    float4 *__restrict__ out, int block0) {
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int base = (block0 + (int)blockIdx.x) * (WAVES * kWave * K) + wave * kWave + lane;
  int zero = 0;
  if constexpr (MODE == 1) asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
  float xi[K], yi[K], zi[K], ax[K], ay[K], az[K];
#pragma unroll
  for (int q = 0; q < K; ++q) {
    const int i = base + q * WAVES * kWave;
    const float4 b = pm[i0 + (i < ni ? i : ni - 1)];
    xi[q] = b.x;
    yi[q] = b.y;
    zi[q] = b.z;
    ax[q] = 0.0f;
    ay[q] = 0.0f;
    az[q] = 0.0f;
  }
  for (int j0 = 0; j0 < n; j0 += T) {
    const int cnt = min(T, n - j0);
    float px[K], py[K], pz[K];
#pragma unroll
    for (int q = 0; q < K; ++q) {
      px[q] = 0.0f;
      py[q] = 0.0f;
      pz[q] = 0.0f;
    }
#pragma unroll 4
    for (int jj = 0; jj < cnt; ++jj) {
      const float4 b = pm[j0 + jj + zero];
#pragma unroll
      for (int q = 0; q < K; ++q)
        pair_accel(b.x, b.y, b.z, b.w, xi[q], yi[q], zi[q], eps2, px[q], py[q], pz[q]);
    }
#pragma unroll
    for (int q = 0; q < K; ++q) {
      ax[q] += px[q];
      ay[q] += py[q];
      az[q] += pz[q];
    }
  }
#pragma unroll
  for (int q = 0; q < K; ++q) {
    const int i = base + q * WAVES * kWave;
    if (i < ni) out[i] = make_float4(G * ax[q], G * ay[q], G * az[q], 0.0f);
  }
}

template <int K, int T, int WAVES, int MODE, int OCC>
static hipError_t launch_stream(const float *posmass, float *accel, int n, int i0, int ni,
                                float G, float eps2, hipStream_t stream) {
  const int per_block = WAVES * kWave * K;
  const int blocks = (ni + per_block - 1) / per_block;
  const int cap = (int)launch_block_cap(WAVES * kWave);
  for (int b0 = 0; b0 < blocks; b0 += cap) {
    hipLaunchKernelGGL((force_stream_kernel<K, T, WAVES, MODE, OCC>),
                       dim3(blocks - b0 < cap ? blocks - b0 : cap), dim3(WAVES * kWave), 0, stream,
                       reinterpret_cast<const float4 *>(posmass), n, i0, ni, G, eps2,
                       reinterpret_cast<float4 *>(accel), b0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int K, int T, int WAVES, int S, int U, int OCC, int LG, class L, bool POT = false>
static hipError_t launch_tile(const L &lay, int n, int i0, int ni, float G, float eps2,
                              hipStream_t stream) {
  constexpr int GW = WAVES / S;
  const int per_block = GW * (kWave / LG) * K;
  const int blocks = (ni + per_block - 1) / per_block;
  const int n_tiles = (n + T - 1) / T;
  const int tiles_per_part = (n_tiles + S - 1) / S;
  const int cap = (int)launch_block_cap(WAVES * kWave);
  for (int b0 = 0; b0 < blocks; b0 += cap) {
    hipLaunchKernelGGL((force_tile_kernel<K, T, WAVES, S, U, OCC, L, POT, LG>),
                       dim3(blocks - b0 < cap ? blocks - b0 : cap), dim3(WAVES * kWave), 0, stream,
                       lay, n, i0, ni, n_tiles, tiles_per_part, G, eps2, b0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// (id, K, T, waves, S, unroll, occupancy target, lane groups).  Ids are part
// of the ABI (nbody_accel_variant):
//  0  one i-body per lane, 64 i-bodies per block, j split 16 ways over 16
//     waves (the small-n shape without lane groups);
//  1  2 i-bodies per lane, 8-wave blocks in 2 j parts, a register budget that
//     fits 8 waves per SIMD (1024 blocks at 2^20);
//  2-4  variant 1 with the inner j loop unrolled 1, 2 and 8 times instead of
//     4: the unroll sweep (the tunable of the CUDA Handbook's Table 14-2);
//  5  2 i-bodies per lane in 4-wave blocks without a j split: the LDS twin of
//     the LDS-free variants 6 and 7 (same K, T and j order, so bitwise equal);
//  8  the library's choice above 32768 bodies: 2 i-bodies per lane in 2
//     lane groups, 64 i-bodies per 16-wave block, j split 16 ways, tiles of
//     128;
//  9  variant 8 with tiles of 64 (a comparison point);
// 10  the choice up to 32768 bodies: variant 8 with 4 lane groups (32
//     i-bodies per block, twice the waves).
// Earlier tilings (1 to 8 i-bodies per lane, tiles of 64 to 512, 4 to 16
// waves, j splits of 1 to 16, 1 to 4 lane groups) were measured on MI355X
// and are not kept.
#define NBODY_FORCE_VARIANTS(X)  \
  X(0, 1, 64, 16, 16, 4, 0, 1)   \
  X(1, 2, 256, 8, 2, 4, 8, 1)    \
  X(2, 2, 256, 8, 2, 1, 8, 1)    \
  X(3, 2, 256, 8, 2, 2, 8, 1)    \
  X(4, 2, 256, 8, 2, 8, 8, 1)    \
  X(5, 2, 256, 4, 1, 4, 0, 1)    \
  X(8, 2, 128, 16, 16, 4, 8, 2)  \
  X(9, 2, 64, 16, 16, 4, 8, 2)   \
  X(10, 2, 128, 16, 16, 4, 8, 4)

// LDS-free variants: (id, K, T, waves, mode, occupancy target); mode 0 =
// scalar loads of j, 1 = vector loads of one address per wave.
#define NBODY_STREAM_VARIANTS(X) \
  X(6, 2, 256, 4, 0, 0)          \
  X(7, 2, 256, 4, 1, 0)

// Ids run 0 .. force_variant_count() - 1 over both tables.
const ForceVariant *force_variant(int v) {
  switch (v) {
#define X(id, K, T, W, S, U, OCC, LG)                      \
  case id: {                                               \
    static const ForceVariant f{K, T, W, S, U, 0, LG};     \
    return &f;                                             \
  }
    NBODY_FORCE_VARIANTS(X)
#undef X
#define X(id, K, T, W, MODE, OCC)                          \
  case id: {                                               \
    static const ForceVariant f{K, T, W, 1, 4, 1 + MODE, 1}; \
    return &f;                                             \
  }
    NBODY_STREAM_VARIANTS(X)
#undef X
    default:
      return nullptr;
  }
}

int force_variant_count() {
  int count = 0;
#define X(...) ++count;
  NBODY_FORCE_VARIANTS(X)
  NBODY_STREAM_VARIANTS(X)
#undef X
  return count;
}

// Measured on MI355X (force-pass sweeps, variants interleaved on one box,
// HIP events around each call).  Up to 32768 bodies variant 10 (4 lane
// groups, 32 i-bodies per block) makes the most waves and is fastest:
// 17.2 us at 4096 (variant 0: 24.9), 30.1 us at 8192 (45.1), 85.6 us at
// 16384 (86.7), 183 us at 24576 (232; there 64-body blocks leave half the
// CUs with one block).  From 32768 on variant 8 (2 lane groups, 64 i-bodies
// per block) is the fastest or within 1 % of it: 4.60 ms at 131072 (variant
// 0: 4.73), 268.5 ms at 1,000,003 (variant 1: 279.0), 289.4 ms at 2^20
// (variant 1: 291.4); variant 1's 512-body blocks fill whole rounds only
// near powers of two.
int force_variant_for_n(int64_t n) { return n <= 32768 ? 10 : 8; }

template <class L>
static hipError_t dispatch(int v, const L &lay, int n, int i0, int ni, float G, float eps2,
                           hipStream_t stream) {
  switch (v) {
#define X(id, K, T, W, S, U, OCC, LG) \
  case id:                            \
    return launch_tile<K, T, W, S, U, OCC, LG>(lay, n, i0, ni, G, eps2, stream);
    NBODY_FORCE_VARIANTS(X)
#undef X
    default:
      return hipErrorInvalidValue;
  }
}

// Variants compiled with the potential sum (the ones force_variant_for_n
// picks).
#define NBODY_POT_VARIANTS(X)   \
  X(8, 2, 128, 16, 16, 4, 8, 2) \
  X(10, 2, 128, 16, 16, 4, 8, 4)

hipError_t launch_force_potential(const float *posmass, int n, float G, float eps2,
                                  float *accel, hipStream_t stream) {
  LayoutAos4 lay{reinterpret_cast<const float4 *>(posmass), reinterpret_cast<float4 *>(accel)};
  switch (force_variant_for_n(n)) {
#define X(id, K, T, W, S, U, OCC, LG) \
  case id:                            \
    return launch_tile<K, T, W, S, U, OCC, LG, LayoutAos4, true>(lay, n, 0, n, G, eps2, stream);
    NBODY_POT_VARIANTS(X)
#undef X
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t launch_force(int variant, Layout layout, const BodyArrays &b, int n, int i0, int ni,
                        float G, float eps2, hipStream_t stream) {
  const ForceVariant *fv = force_variant(variant);
  if (fv && fv->staging != 0) {
    if (layout != Layout::Aos4) return hipErrorInvalidValue;
    switch (variant) {
#define X(id, K, T, W, MODE, OCC) \
  case id:                        \
    return launch_stream<K, T, W, MODE, OCC>(b.posmass, b.accel4, n, i0, ni, G, eps2, stream);
      NBODY_STREAM_VARIANTS(X)
#undef X
      default:
        return hipErrorInvalidValue;
    }
  }
  switch (layout) {
    case Layout::Aos4: {
      LayoutAos4 lay{reinterpret_cast<const float4 *>(b.posmass),
                     reinterpret_cast<float4 *>(b.accel4)};
      return dispatch(variant, lay, n, i0, ni, G, eps2, stream);
    }
    case Layout::Aos3: {
      LayoutAos3 lay{b.pos3, b.mass, b.accel3};
      return dispatch(variant, lay, n, i0, ni, G, eps2, stream);
    }
    case Layout::Soa: {
      LayoutSoa lay{b.x, b.y, b.z, b.m, b.ax, b.ay, b.az};
      return dispatch(variant, lay, n, i0, ni, G, eps2, stream);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace nbody
