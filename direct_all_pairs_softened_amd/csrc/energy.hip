// Energy and momentum: K = sum m v^2 / 2, W = -G sum_{i<j} m_i m_j /
// sqrt(r^2 + eps^2), P = sum m v, M = sum m.  (The pages give no energy
// formula; W is the softened pair potential whose negative gradient is the
// README's section 1.2 acceleration, each pair counted once.)
//
// Pass 1 (energy_partial_kernel): an all-pairs potential pass with the force
// kernel's LDS tiling, one i-body per lane.  Pair terms are fp32; each j-tile
// partial is added to a per-body fp64 running sum.  Then every body's
// (K_i, W_i = -G m_i phi_i / 2, m_i v_i, m_i) is formed in fp64 and the block
// adds them in a fixed tree order.  Pass 2 (energy_final_kernel, one block)
// adds the block partials in a fixed order.  No atomics anywhere, so the
// result is bitwise reproducible -- the shared-memory halving tree of the
// atomics tutorial (CUDA programming part 9, section 1) without its atomic
// tail, and the atomic-free second pass of README section 3.3.
#include "nbody_common.hpp"
#include "nbody_internal.hpp"

namespace nbody {

namespace {

constexpr int kEnergyFields = 6;  // K, W, Px, Py, Pz, M
constexpr int kFinalThreads = 256;

template <int T, int WAVES, int S>
__global__ __launch_bounds__(WAVES *kWave) void energy_partial_kernel(
    const float4 *__restrict__ pm, const float4 *__restrict__ vel, int n, int n_tiles,
    int tiles_per_part, float G, float eps2, double *__restrict__ block_out) {
  constexpr int GW = WAVES / S;
  constexpr int NTHREADS = WAVES * kWave;
  constexpr int LOADS = (S * T) / NTHREADS;
  constexpr int PER_BLOCK = GW * kWave;
  static_assert(WAVES % S == 0 && (S * T) % NTHREADS == 0, "bad energy tiling");
  static_assert((S - 1) * GW * kWave * 8 <= 2 * S * T * 16, "part scratch must fit");
  __shared__ float4 tile[2][S * T];
  __shared__ double red[kEnergyFields][PER_BLOCK];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int part = wave / GW;
  const int grp = wave % GW;
  const int i = blockIdx.x * PER_BLOCK + grp * kWave + lane;
  const float4 me = pm[i < n ? i : n - 1];
  double phi = 0.0;

  // The padding test is kept apart from the load and applied in stash(), so
  // the global load stays in flight across the current tile's arithmetic.
  float4 reg[LOADS];
  bool real[LOADS];
  auto fetch = [&](int step) {
#pragma unroll
    for (int r = 0; r < LOADS; ++r) {
      const int e = tid + r * NTHREADS;
      const int j = ((e / T) * tiles_per_part + step) * T + (e % T);
      reg[r] = pm[j < n ? j : n - 1];
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
    const int t = part * tiles_per_part + step;
    if (t < n_tiles) {
      const float4 *tp = &tile[cur][part * T];
      const int j0 = t * T;
      float p = 0.0f;
#pragma unroll 4
      for (int jj = 0; jj < T; ++jj) {
        const float4 b = tp[jj];
        const float inv = pair_rsq(b.x, b.y, b.z, me.x, me.y, me.z, eps2);
        const float mj = (j0 + jj == i) ? 0.0f : b.w;
        p = __builtin_fmaf(mj, inv, p);
      }
      phi += (double)p;
    }
    if (more) stash(cur ^ 1);
  }

  if constexpr (S > 1) {
    __syncthreads();
    double *sc = reinterpret_cast<double *>(&tile[0][0]);
    if (part > 0) sc[((part - 1) * GW + grp) * kWave + lane] = phi;
    __syncthreads();
    if (part == 0)
      for (int p = 1; p < S; ++p) phi += sc[((p - 1) * GW + grp) * kWave + lane];
  }

  if (part == 0) {
    double f[kEnergyFields] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
    if (i < n) {
      const float4 v = vel[i];
      const double m = (double)me.w;
      const double vx = v.x, vy = v.y, vz = v.z;
      f[0] = 0.5 * m * (vx * vx + vy * vy + vz * vz);
      f[1] = -0.5 * (double)G * m * phi;
      f[2] = m * vx;
      f[3] = m * vy;
      f[4] = m * vz;
      f[5] = m;
    }
    const int t = grp * kWave + lane;  // part-0 waves are waves 0 .. GW-1
#pragma unroll
    for (int c = 0; c < kEnergyFields; ++c) red[c][t] = f[c];
  }
  __syncthreads();
  for (int s = PER_BLOCK / 2; s > 0; s >>= 1) {
    if (tid < s) {
#pragma unroll
      for (int c = 0; c < kEnergyFields; ++c) red[c][tid] += red[c][tid + s];
    }
    __syncthreads();
  }
  if (tid < kEnergyFields) block_out[(size_t)blockIdx.x * 8 + tid] = red[tid][0];
}

__global__ __launch_bounds__(kFinalThreads) void energy_final_kernel(
    const double *__restrict__ block_out, int nblocks, double *__restrict__ stats) {
  __shared__ double red[kEnergyFields][kFinalThreads];
  const int tid = threadIdx.x;
  double f[kEnergyFields] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
  for (int b = tid; b < nblocks; b += kFinalThreads) {
#pragma unroll
    for (int c = 0; c < kEnergyFields; ++c) f[c] += block_out[(size_t)b * 8 + c];
  }
#pragma unroll
  for (int c = 0; c < kEnergyFields; ++c) red[c][tid] = f[c];
  __syncthreads();
  for (int s = kFinalThreads / 2; s > 0; s >>= 1) {
    if (tid < s) {
#pragma unroll
      for (int c = 0; c < kEnergyFields; ++c) red[c][tid] += red[c][tid + s];
    }
    __syncthreads();
  }
  if (tid == 0) {
    const double K = red[0][0], W = red[1][0];
    stats[0] = K;
    stats[1] = W;
    stats[2] = K + W;
    stats[3] = red[2][0];
    stats[4] = red[3][0];
    stats[5] = red[4][0];
    stats[6] = red[5][0];
    stats[7] = 0.0;
  }
}

// O(N) energy from per-body potentials Phi_i (accel.w of the potential
// force pass): K_i = m v^2 / 2, W_i = m_i Phi_i / 2, P, M; fp64 tree per
// block, then energy_final_kernel.
constexpr int kFromPotThreads = 256;

__global__ __launch_bounds__(kFromPotThreads) void energy_from_potential_kernel(
    const float4 *__restrict__ pm, const float4 *__restrict__ vel,
    const float4 *__restrict__ acc, int n, double *__restrict__ block_out) {
  __shared__ double red[kEnergyFields][kFromPotThreads];
  const int tid = threadIdx.x;
  const int i = blockIdx.x * kFromPotThreads + tid;
  double f[kEnergyFields] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
  if (i < n) {
    const float4 b = pm[i], v = vel[i], a = acc[i];
    const double m = (double)b.w;
    const double vx = v.x, vy = v.y, vz = v.z;
    f[0] = 0.5 * m * (vx * vx + vy * vy + vz * vz);
    f[1] = 0.5 * m * (double)a.w;
    f[2] = m * vx;
    f[3] = m * vy;
    f[4] = m * vz;
    f[5] = m;
  }
#pragma unroll
  for (int c = 0; c < kEnergyFields; ++c) red[c][tid] = f[c];
  __syncthreads();
  for (int s = kFromPotThreads / 2; s > 0; s >>= 1) {
    if (tid < s) {
#pragma unroll
      for (int c = 0; c < kEnergyFields; ++c) red[c][tid] += red[c][tid + s];
    }
    __syncthreads();
  }
  if (tid < kEnergyFields) block_out[(size_t)blockIdx.x * 8 + tid] = red[tid][0];
}

struct EnergyShape {
  int T, waves, split;
};

EnergyShape energy_shape(int64_t n) {
  if (n <= 65536) return {64, 16, 16};  // 64 bodies per block, j split 16 ways
  return {256, 4, 1};                   // 256 bodies per block
}

int energy_blocks(int64_t n) {
  const EnergyShape s = energy_shape(n);
  const int per_block = (s.waves / s.split) * kWave;
  return (int)((n + per_block - 1) / per_block);
}

template <int T, int WAVES, int S>
hipError_t launch_partial(const float4 *pm, const float4 *vel, int n, float G, float eps2,
                          double *block_out, hipStream_t stream) {
  const int per_block = (WAVES / S) * kWave;
  const int blocks = (n + per_block - 1) / per_block;
  const int n_tiles = (n + T - 1) / T;
  const int tiles_per_part = (n_tiles + S - 1) / S;
  hipLaunchKernelGGL((energy_partial_kernel<T, WAVES, S>), dim3(blocks), dim3(WAVES * kWave), 0,
                     stream, pm, vel, n, n_tiles, tiles_per_part, G, eps2, block_out);
  return hipGetLastError();
}

}  // namespace

size_t energy_from_potential_workspace_bytes(int64_t n) {
  if (n <= 0) return 0;
  return (size_t)((n + kFromPotThreads - 1) / kFromPotThreads) * 8 * sizeof(double);
}

hipError_t launch_energy_from_potential(const float *posmass, const float *vel,
                                        const float *accel, int n, void *workspace,
                                        double *stats, hipStream_t stream) {
  const int blocks = (n + kFromPotThreads - 1) / kFromPotThreads;
  double *block_out = reinterpret_cast<double *>(workspace);
  hipLaunchKernelGGL(energy_from_potential_kernel, dim3(blocks), dim3(kFromPotThreads), 0, stream,
                     reinterpret_cast<const float4 *>(posmass),
                     reinterpret_cast<const float4 *>(vel), reinterpret_cast<const float4 *>(accel),
                     n, block_out);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(energy_final_kernel, dim3(1), dim3(kFinalThreads), 0, stream, block_out,
                     blocks, stats);
  return hipGetLastError();
}

size_t energy_workspace_bytes(int64_t n) {
  if (n <= 0) return 0;
  return (size_t)energy_blocks(n) * 8 * sizeof(double);
}

hipError_t launch_energy(const float *posmass, const float *vel, int n, float G, float eps2,
                         void *workspace, double *stats, hipStream_t stream) {
  const float4 *pm = reinterpret_cast<const float4 *>(posmass);
  const float4 *v = reinterpret_cast<const float4 *>(vel);
  double *block_out = reinterpret_cast<double *>(workspace);
  const EnergyShape s = energy_shape(n);
  hipError_t e;
  if (s.split == 16)
    e = launch_partial<64, 16, 16>(pm, v, n, G, eps2, block_out, stream);
  else
    e = launch_partial<256, 4, 1>(pm, v, n, G, eps2, block_out, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(energy_final_kernel, dim3(1), dim3(kFinalThreads), 0, stream, block_out,
                     energy_blocks(n), stats);
  return hipGetLastError();
}

}  // namespace nbody
