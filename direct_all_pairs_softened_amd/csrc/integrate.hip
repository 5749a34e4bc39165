// Leapfrog kick / drift kernels (section 1.3 of the "CUDA N-Body Simulation"
// README: v += (dt/2) a, then x += dt v), kept apart from the force kernel:
// positions are only written once every block of the force pass has read
// them.  One lane per body, 16-byte loads and stores; bandwidth-bound
// (80 bytes per body for kick+drift, 48 for a kick alone).
#include "nbody_common.hpp"
#include "nbody_internal.hpp"

namespace nbody {

namespace {

constexpr int kIntThreads = 256;

__global__ __launch_bounds__(kIntThreads) void leapfrog_kernel(float4 *__restrict__ pm,
                                                               float4 *__restrict__ vel,
                                                               const float4 *__restrict__ acc,
                                                               int n, float dt, float h) {
  const int i = blockIdx.x * kIntThreads + threadIdx.x;
  if (i >= n) return;
  float4 x = pm[i];
  float4 v = vel[i];
  const float4 a = acc[i];
  v.x = __builtin_fmaf(h, a.x, v.x);
  v.y = __builtin_fmaf(h, a.y, v.y);
  v.z = __builtin_fmaf(h, a.z, v.z);
  x.x = __builtin_fmaf(dt, v.x, x.x);
  x.y = __builtin_fmaf(dt, v.y, x.y);
  x.z = __builtin_fmaf(dt, v.z, x.z);
  pm[i] = x;   // x.w (mass) written back unchanged
  vel[i] = v;  // v.w written back unchanged
}

__global__ __launch_bounds__(kIntThreads) void kick_kernel(float4 *__restrict__ vel,
                                                           const float4 *__restrict__ acc,
                                                           int n, float h) {
  const int i = blockIdx.x * kIntThreads + threadIdx.x;
  if (i >= n) return;
  float4 v = vel[i];
  const float4 a = acc[i];
  v.x = __builtin_fmaf(h, a.x, v.x);
  v.y = __builtin_fmaf(h, a.y, v.y);
  v.z = __builtin_fmaf(h, a.z, v.z);
  vel[i] = v;
}

// The closing half-kick of one step and the kick-drift of the next, which
// use the same accelerations, in one pass over the bodies: the same
// operations in the same order as kick_kernel then leapfrog_kernel (each
// half-kick a separate multiply-add), so the result is bitwise theirs.
__global__ __launch_bounds__(kIntThreads) void kick_leapfrog_kernel(float4 *__restrict__ pm,
                                                                    float4 *__restrict__ vel,
                                                                    const float4 *__restrict__ acc,
                                                                    int n, float dt, float h) {
  const int i = blockIdx.x * kIntThreads + threadIdx.x;
  if (i >= n) return;
  float4 x = pm[i];
  float4 v = vel[i];
  const float4 a = acc[i];
  v.x = __builtin_fmaf(h, a.x, v.x);
  v.y = __builtin_fmaf(h, a.y, v.y);
  v.z = __builtin_fmaf(h, a.z, v.z);
  v.x = __builtin_fmaf(h, a.x, v.x);
  v.y = __builtin_fmaf(h, a.y, v.y);
  v.z = __builtin_fmaf(h, a.z, v.z);
  x.x = __builtin_fmaf(dt, v.x, x.x);
  x.y = __builtin_fmaf(dt, v.y, x.y);
  x.z = __builtin_fmaf(dt, v.z, x.z);
  pm[i] = x;
  vel[i] = v;
}

}  // namespace

hipError_t launch_kick_leapfrog(float *posmass, float *vel, const float *accel, float dt, int n,
                                hipStream_t stream) {
  hipLaunchKernelGGL(kick_leapfrog_kernel, dim3((n + kIntThreads - 1) / kIntThreads),
                     dim3(kIntThreads), 0, stream, reinterpret_cast<float4 *>(posmass),
                     reinterpret_cast<float4 *>(vel), reinterpret_cast<const float4 *>(accel),
                     n, dt, 0.5f * dt);
  return hipGetLastError();
}

hipError_t launch_leapfrog(float *posmass, float *vel, const float *accel, float dt, int n,
                           hipStream_t stream) {
  hipLaunchKernelGGL(leapfrog_kernel, dim3((n + kIntThreads - 1) / kIntThreads),
                     dim3(kIntThreads), 0, stream, reinterpret_cast<float4 *>(posmass),
                     reinterpret_cast<float4 *>(vel), reinterpret_cast<const float4 *>(accel),
                     n, dt, 0.5f * dt);
  return hipGetLastError();
}

hipError_t launch_kick(float *vel, const float *accel, float h, int n, hipStream_t stream) {
  hipLaunchKernelGGL(kick_kernel, dim3((n + kIntThreads - 1) / kIntThreads), dim3(kIntThreads),
                     0, stream, reinterpret_cast<float4 *>(vel),
                     reinterpret_cast<const float4 *>(accel), n, h);
  return hipGetLastError();
}

}  // namespace nbody
