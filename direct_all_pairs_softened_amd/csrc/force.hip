// Force pass: LDS-tiled all-pairs softened gravity for gfx950.
//
// Decomposition (the tiled scheme of "Cuda Nbody Notes" and of section 3.1
// of the "CUDA N-Body Simulation" README, rebuilt for 64-wide wavefronts):
//  - each lane keeps K i-bodies and their accumulators in VGPRs;
//  - a block of `waves` wavefronts stages j-bodies in LDS tiles of T bodies;
//    every lane of a wave reads the same LDS address, which the LDS serves as
//    a broadcast (the CUDA Handbook's shared-memory page makes the same point
//    for warps);
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
template <int K, int T, int WAVES, int S, int U, int OCC, class L, bool POT = false>
__global__ __launch_bounds__(WAVES *kWave)
__attribute__((amdgpu_waves_per_eu(OCC > 0 ? OCC : 1))) void force_tile_kernel(
    L lay, int n, int i0, int ni, int n_tiles, int tiles_per_part, float G, float eps2) {
  constexpr int GW = WAVES / S;            // i-groups (waves) per part
  constexpr int NTHREADS = WAVES * kWave;  // threads per block
  constexpr int LOADS = (S * T) / NTHREADS;
  static_assert(WAVES % S == 0, "waves must be a multiple of the split");
  static_assert((S * T) % NTHREADS == 0, "staged bodies must divide evenly over threads");
  static_assert(S == 1 || GW * K * (POT ? 4 : 3) * kWave <= 2 * S * T * 4,
                "one part's sums must fit in the tile buffers");
  __shared__ float4 tile[2][S * T];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int part = wave / GW;
  const int grp = wave % GW;
  const int base = blockIdx.x * (GW * kWave * K) + grp * kWave + lane;

  float xi[K], yi[K], zi[K], ax[K], ay[K], az[K], ap[K];
#pragma unroll
  for (int q = 0; q < K; ++q) {
    const int i = base + q * GW * kWave;
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
      for (int jj = 0; jj < T; ++jj) {
        const float4 b = tp[jj];
#pragma unroll
        for (int q = 0; q < K; ++q) {
          if constexpr (POT) {
            const float mp = (j0 + jj == i0 + base + q * GW * kWave) ? 0.0f : b.w;
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

  if (part == 0) {
#pragma unroll
    for (int q = 0; q < K; ++q) {
      const int i = base + q * GW * kWave;
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
    float4 *__restrict__ out) {
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int base = blockIdx.x * (WAVES * kWave * K) + wave * kWave + lane;
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
  hipLaunchKernelGGL((force_stream_kernel<K, T, WAVES, MODE, OCC>), dim3(blocks),
                     dim3(WAVES * kWave), 0, stream, reinterpret_cast<const float4 *>(posmass), n,
                     i0, ni, G, eps2, reinterpret_cast<float4 *>(accel));
  return hipGetLastError();
}

template <int K, int T, int WAVES, int S, int U, int OCC, class L, bool POT = false>
static hipError_t launch_tile(const L &lay, int n, int i0, int ni, float G, float eps2,
                              hipStream_t stream) {
  constexpr int GW = WAVES / S;
  const int per_block = GW * kWave * K;
  const int blocks = (ni + per_block - 1) / per_block;
  const int n_tiles = (n + T - 1) / T;
  const int tiles_per_part = (n_tiles + S - 1) / S;
  hipLaunchKernelGGL((force_tile_kernel<K, T, WAVES, S, U, OCC, L, POT>), dim3(blocks),
                     dim3(WAVES * kWave), 0, stream, lay, n, i0, ni, n_tiles, tiles_per_part, G,
                     eps2);
  return hipGetLastError();
}

// (id, K, T, waves, S, unroll, occupancy target).  Ids are part of the ABI
// (nbody_accel_variant):
//  0  the library's choice up to 2e5 bodies: 64 i-bodies per block, j split
//     16 ways over 16 waves;
//  1  the choice above: 2 i-bodies per lane, 8-wave blocks in 2 j parts, a
//     register budget that fits 8 waves per SIMD (1024 blocks at 2^20);
//  2-4  variant 1 with the inner j loop unrolled 1, 2 and 8 times instead of
//     4: the unroll sweep (the tunable of the CUDA Handbook's Table 14-2);
//  5  2 i-bodies per lane in 4-wave blocks without a j split: the LDS twin of
//     the LDS-free variants 6 and 7 (same K, T and j order, so bitwise equal).
// Earlier tilings (1 to 8 i-bodies per lane, tiles of 64 to 512, 4 to 16
// waves, j splits of 1 to 16) were measured on MI355X and are not kept.
#define NBODY_FORCE_VARIANTS(X)  \
  X(0, 1, 64, 16, 16, 4, 0)      \
  X(1, 2, 256, 8, 2, 4, 8)       \
  X(2, 2, 256, 8, 2, 1, 8)       \
  X(3, 2, 256, 8, 2, 2, 8)       \
  X(4, 2, 256, 8, 2, 8, 8)       \
  X(5, 2, 256, 4, 1, 4, 0)

// LDS-free variants: (id, K, T, waves, mode, occupancy target); mode 0 =
// scalar loads of j, 1 = vector loads of one address per wave.
#define NBODY_STREAM_VARIANTS(X) \
  X(6, 2, 256, 4, 0, 0)          \
  X(7, 2, 256, 4, 1, 0)

static const ForceVariant kVariants[] = {
#define X(id, K, T, W, S, U, OCC) {K, T, W, S, U, 0},
    NBODY_FORCE_VARIANTS(X)
#undef X
#define X(id, K, T, W, MODE, OCC) {K, T, W, 1, 4, 1 + MODE},
        NBODY_STREAM_VARIANTS(X)
#undef X
};

int force_variant_count() { return (int)(sizeof(kVariants) / sizeof(kVariants[0])); }

const ForceVariant *force_variant(int v) {
  return (v >= 0 && v < force_variant_count()) ? &kVariants[v] : nullptr;
}

// Measured on MI355X (force-pass sweeps over every variant): small and
// medium n want one body per lane and a 16-way j split, so that every SIMD
// holds several waves; from a few hundred thousand bodies on, two bodies per
// lane in 8-wave blocks (two j parts) with a VGPR budget that fits 8 waves
// per SIMD is fastest.
int force_variant_for_n(int64_t n) {
  if (n <= 200000) return 0;  // 64 i per block, j split 16 ways
  return 1;                   // 512 i per block, j split 2 ways, 8 waves/SIMD
}

template <class L>
static hipError_t dispatch(int v, const L &lay, int n, int i0, int ni, float G, float eps2,
                           hipStream_t stream) {
  switch (v) {
#define X(id, K, T, W, S, U, OCC) \
  case id:                        \
    return launch_tile<K, T, W, S, U, OCC>(lay, n, i0, ni, G, eps2, stream);
    NBODY_FORCE_VARIANTS(X)
#undef X
    default:
      return hipErrorInvalidValue;
  }
}

// Variants compiled with the potential sum (the ones force_variant_for_n
// picks).
#define NBODY_POT_VARIANTS(X) \
  X(0, 1, 64, 16, 16, 4, 0)   \
  X(1, 2, 256, 8, 2, 4, 8)

hipError_t launch_force_potential(const float *posmass, int n, float G, float eps2,
                                  float *accel, hipStream_t stream) {
  LayoutAos4 lay{reinterpret_cast<const float4 *>(posmass), reinterpret_cast<float4 *>(accel)};
  switch (force_variant_for_n(n)) {
#define X(id, K, T, W, S, U, OCC) \
  case id:                        \
    return launch_tile<K, T, W, S, U, OCC, LayoutAos4, true>(lay, n, 0, n, G, eps2, stream);
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
