// Energy and momentum: K = sum m v^2 / 2, W = -G sum_{i<j} m_i m_j /
// sqrt(r^2 + eps^2), P = sum m v, M = sum m.  (The pages give no energy
// formula; W is the softened pair potential whose negative gradient is the
// README's section 1.2 acceleration, each pair counted once.)
//
// Three passes, no atomics, every sum in a fixed order (bitwise reproducible):
//  1. energy_bodies_kernel: per body K_i, m_i v_i, m_i in fp64, added in a
//     fixed halving tree per block of 256 bodies (the shared-memory tree of
//     the atomics tutorial, CUDA programming part 9, section 1, without its
//     atomic tail).  The same kernel with the potential flag takes
//     W_i = m_i Phi_i / 2 from accel.w (nbody_energy_from_potential).
//  2. energy_pairs_kernel: the pair sum of W over panel-pair tasks (I <= J),
//     the panel-pair scheme of the pair-symmetric force pass: each lane keeps
//     K i-bodies, every unordered pair is met once (in a diagonal task,
//     twice, and halved; the j = i pair is skipped by an index test).  The
//     pair potential is symmetric, so no j-side sum is needed: each wave
//     stages 64 j-bodies in its LDS tile and all lanes read the same one per
//     step (a broadcast read, no lane rotation).  Per (lane, i-body) the
//     terms m_j / sqrt(r^2 + eps^2) of a 64-body sweep are summed in fp32 in
//     ascending j, multiplied by m_i and added in fp64; lanes are added in a
//     fixed tree.  One fp64 value per task.
//  3. energy_final_kernel: block sums and task sums in fixed orders.
#include "nbody_common.hpp"
#include "nbody_internal.hpp"

#include <mutex>

namespace nbody {

namespace {

constexpr int kEnergyFields = 6;  // K, W, Px, Py, Pz, M
constexpr int kBodyThreads = 256;
constexpr int kFinalThreads = 256;
constexpr int kPairK = 8;  // i-bodies per lane in the pair pass
constexpr int kPairW = 4;  // waves per block in the pair pass
constexpr int kPairPanel = kPairK * kPairW * kWave;

template <bool WITH_POTENTIAL>
__global__ __launch_bounds__(kBodyThreads) void energy_bodies_kernel(
    const float4 *__restrict__ pm, const float4 *__restrict__ vel,
    const float4 *__restrict__ acc, int n, double *__restrict__ block_out) {
  __shared__ double red[kEnergyFields][kBodyThreads];
  const int tid = threadIdx.x;
  const int i = blockIdx.x * kBodyThreads + tid;
  double f[kEnergyFields] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
  if (i < n) {
    const float4 b = pm[i], v = vel[i];
    const double m = (double)b.w;
    const double vx = v.x, vy = v.y, vz = v.z;
    f[0] = 0.5 * m * (vx * vx + vy * vy + vz * vz);
    if constexpr (WITH_POTENTIAL) f[1] = 0.5 * m * (double)acc[i].w;
    f[2] = m * vx;
    f[3] = m * vy;
    f[4] = m * vz;
    f[5] = m;
  }
#pragma unroll
  for (int c = 0; c < kEnergyFields; ++c) red[c][tid] = f[c];
  __syncthreads();
  for (int s = kBodyThreads / 2; s > 0; s >>= 1) {
    if (tid < s) {
#pragma unroll
      for (int c = 0; c < kEnergyFields; ++c) red[c][tid] += red[c][tid + s];
    }
    __syncthreads();
  }
  if (tid < kEnergyFields) block_out[(size_t)blockIdx.x * 8 + tid] = red[tid][0];
}

template <bool DIAG>
__device__ __forceinline__ double pair_potential_task(const float4 *__restrict__ pm, int n, int I,
                                                      int J, float eps2, float4 *jt) {
  constexpr int K = kPairK, B = kPairPanel, NG = B / kWave;
  constexpr int U = 2;  // steps per unrolled block
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  float xi[K], yi[K], zi[K], mi[K];
#pragma unroll
  for (int q = 0; q < K; ++q) {
    const int i = I * B + wave * (kWave * K) + q * kWave + lane;
    const float4 b = pm[i < n ? i : n - 1];
    xi[q] = b.x;
    yi[q] = b.y;
    zi[q] = b.z;
    mi[q] = i < n ? b.w : 0.0f;
  }
  double acc = 0.0;
  for (int g = 0; g < NG; ++g) {
    const int j = J * B + g * kWave + lane;
    const float4 b = pm[j < n ? j : n - 1];
    jt[lane] = make_float4(b.x, b.y, b.z, j < n ? b.w : 0.0f);
    // every lane reads what the others wrote: keep the LDS accesses on
    // their side of this point (one wave's LDS instructions run in order)
    asm volatile("" ::: "memory");
    float s[K];
#pragma unroll
    for (int q = 0; q < K; ++q) s[q] = 0.0f;
    for (int s0 = 0; s0 < kWave; s0 += U) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float4 y = jt[s0 + u];  // the same j-body for all lanes (broadcast)
        // the K pairs of the step in phases (all differences, all d^2, all
        // rsq, then the sums): K independent chains to issue from, where one
        // pair after the other leaves the VALU waiting on each result
        float dx[K], dy[K], dz[K], w[K];
#pragma unroll
        for (int q = 0; q < K; ++q) {
          dx[q] = y.x - xi[q];
          dy[q] = y.y - yi[q];
          dz[q] = y.z - zi[q];
        }
#pragma unroll
        for (int q = 0; q < K; ++q) w[q] = __builtin_fmaf(dx[q], dx[q], eps2);
#pragma unroll
        for (int q = 0; q < K; ++q) w[q] = __builtin_fmaf(dy[q], dy[q], w[q]);
#pragma unroll
        for (int q = 0; q < K; ++q) w[q] = __builtin_fmaf(dz[q], dz[q], w[q]);
#pragma unroll
        for (int q = 0; q < K; ++q) w[q] = __builtin_amdgcn_rsqf(w[q]);
#pragma unroll
        for (int q = 0; q < K; ++q) {
          float mp = y.w;
          // in a diagonal task lane l meets its own body at step l of the
          // sweep whose j-group is that body's group (wave * K + q)
          if constexpr (DIAG) mp = (g == wave * K + q && s0 + u == lane) ? 0.0f : y.w;
          s[q] = __builtin_fmaf(mp, w[q], s[q]);
        }
      }
    }
    asm volatile("" ::: "memory");
#pragma unroll
    for (int q = 0; q < K; ++q) acc += (double)mi[q] * (double)s[q];
  }
  return acc;
}

// One block per panel pair (I, J), I <= J, in the XCD-aware order of
// PanelOrder: task_out[t] = sum over the pairs of m_i m_j / sqrt(r^2 + eps^2),
// each unordered pair once, t the pair's number in that order.
__global__ __launch_bounds__(kPairW *kWave) void energy_pairs_kernel(
    const float4 *__restrict__ pm, int n, PanelOrder order, float eps2,
    double *__restrict__ task_out) {
  __shared__ double red[kPairW * kWave];
  __shared__ float4 jtile[kPairW * kWave];  // one 64-body j-tile per wave
  int I, J;
  long long t;
  if (!panel_pair_of_block(order, blockIdx.x, I, J, t)) return;  // whole block: no barrier skipped
  const int tid = threadIdx.x;
  float4 *jt = jtile + (tid / kWave) * kWave;
  double acc = I == J ? pair_potential_task<true>(pm, n, I, J, eps2, jt)
                      : pair_potential_task<false>(pm, n, I, J, eps2, jt);
  red[tid] = acc;
  __syncthreads();
  for (int s = kPairW * kWave / 2; s > 0; s >>= 1) {
    if (tid < s) red[tid] += red[tid + s];
    __syncthreads();
  }
  // a diagonal task met every pair twice; halving is exact
  if (tid == 0) task_out[t] = I == J ? 0.5 * red[0] : red[0];
}

__global__ __launch_bounds__(kFinalThreads) void energy_final_kernel(
    const double *__restrict__ block_out, int nblocks, const double *__restrict__ task_out,
    long long ntasks, double G, double *__restrict__ stats) {
  __shared__ double red[kEnergyFields + 1][kFinalThreads];
  const int tid = threadIdx.x;
  double f[kEnergyFields + 1] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
  for (int b = tid; b < nblocks; b += kFinalThreads) {
#pragma unroll
    for (int c = 0; c < kEnergyFields; ++c) f[c] += block_out[(size_t)b * 8 + c];
  }
  for (long long t = tid; t < ntasks; t += kFinalThreads) f[kEnergyFields] += task_out[t];
#pragma unroll
  for (int c = 0; c <= kEnergyFields; ++c) red[c][tid] = f[c];
  __syncthreads();
  for (int s = kFinalThreads / 2; s > 0; s >>= 1) {
    if (tid < s) {
#pragma unroll
      for (int c = 0; c <= kEnergyFields; ++c) red[c][tid] += red[c][tid + s];
    }
    __syncthreads();
  }
  if (tid == 0) {
    // W comes from the bodies pass (potential path) or from the pair sum
    const double K = red[0][0];
    const double W = red[1][0] - G * red[kEnergyFields][0];
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

int body_blocks(int64_t n) { return (int)((n + kBodyThreads - 1) / kBodyThreads); }

long long pair_tasks(int64_t n) {
  const long long P = (n + kPairPanel - 1) / kPairPanel;
  return P * (P + 1) / 2;
}

}  // namespace

size_t energy_from_potential_workspace_bytes(int64_t n) {
  if (n <= 0) return 0;
  return (size_t)body_blocks(n) * 8 * sizeof(double);
}

hipError_t launch_energy_from_potential(const float *posmass, const float *vel,
                                        const float *accel, int n, void *workspace,
                                        double *stats, hipStream_t stream) {
  const int blocks = body_blocks(n);
  double *block_out = reinterpret_cast<double *>(workspace);
  hipLaunchKernelGGL(energy_bodies_kernel<true>, dim3(blocks), dim3(kBodyThreads), 0, stream,
                     reinterpret_cast<const float4 *>(posmass),
                     reinterpret_cast<const float4 *>(vel), reinterpret_cast<const float4 *>(accel),
                     n, block_out);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(energy_final_kernel, dim3(1), dim3(kFinalThreads), 0, stream, block_out,
                     blocks, (const double *)nullptr, 0LL, 0.0, stats);
  return hipGetLastError();
}

size_t energy_workspace_bytes(int64_t n) {
  if (n <= 0) return 0;
  return ((size_t)body_blocks(n) * 8 + (size_t)pair_tasks(n)) * sizeof(double);
}

int64_t energy_pair_tasks(int64_t n) { return n <= 0 ? 0 : pair_tasks(n); }

// Scratch of the allocation-free energy entry point: one copy per GPU, held
// until the process ends.  Host code never uses this name as an address (on
// the host it is only a stand-in for the symbol); it uses the device address
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[kEnergyStaticScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t energy_static_scratch(void **ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_energy(const float *posmass, const float *vel, int n, float G, float eps2,
                         void *workspace, double *stats, hipStream_t stream) {
  const int blocks = body_blocks(n);
  const long long tasks = pair_tasks(n);
  double *block_out = reinterpret_cast<double *>(workspace);
  double *task_out = block_out + (size_t)blocks * 8;
  const float4 *pm = reinterpret_cast<const float4 *>(posmass);
  hipLaunchKernelGGL(energy_bodies_kernel<false>, dim3(blocks), dim3(kBodyThreads), 0, stream, pm,
                     reinterpret_cast<const float4 *>(vel), (const float4 *)nullptr, n,
                     block_out);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long P = (n + kPairPanel - 1) / kPairPanel;
  e = launch_pair_ranges(P, 0, tasks, kPairW * kWave, [&](const PanelOrder &o, long long b) {
    hipLaunchKernelGGL(energy_pairs_kernel, dim3((unsigned)b), dim3(kPairW * kWave), 0, stream,
                       pm, n, o, eps2, task_out);
  });
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(energy_final_kernel, dim3(1), dim3(kFinalThreads), 0, stream, block_out,
                     blocks, task_out, tasks, (double)G, stats);
  return hipGetLastError();
}

}  // namespace nbody
