// Two-pass force decomposition over j chunks: the N x N interaction grid cut
// into (i-block, j-chunk) cells, each writing one partial sum per body, and a
// second, atomic-free pass that adds the chunk partials of every body in
// ascending chunk order.  Sections 3.2 and 3.3 of the "CUDA N-Body
// Simulation" README describe this shape with 32-wide chunks reduced by a
// shared-memory tree; here a lane owns one i-body and walks its chunk
// sequentially (no tree), and the chunk width is a parameter (>= 32).  The
// page notes that the second pass makes the result deterministic for a
// given grid; the same holds here for a given chunk width.
#include "nbody_common.hpp"
#include "nbody_internal.hpp"

namespace nbody {

namespace {

constexpr int kSplitWaves = 4;
constexpr int kSplitThreads = kSplitWaves * kWave;
constexpr int kSplitTile = kSplitThreads;  // LDS sub-tile: one body per thread

// grid = (ceil(n / 256), n_chunks).  partial is float4 [n_chunks][n].
__global__ __launch_bounds__(kSplitThreads) void splitj_partial_kernel(
    const float4 *__restrict__ pm, int n, int j_chunk, float eps2,
    float4 *__restrict__ partial) {
  __shared__ float4 tile[kSplitTile];
  const int tid = threadIdx.x;
  const int i = blockIdx.x * kSplitThreads + tid;
  const float4 me = pm[i < n ? i : n - 1];
  const int c = blockIdx.y;
  const int j0 = c * j_chunk;
  float sx = 0.0f, sy = 0.0f, sz = 0.0f;
  for (int t0 = 0; t0 < j_chunk; t0 += kSplitTile) {
    const int width = min(kSplitTile, j_chunk - t0);  // uniform
    __syncthreads();
    if (tid < width) {
      const int j = j0 + t0 + tid;
      float4 b = pm[j < n ? j : n - 1];
      b.w = j < n ? b.w : 0.0f;
      tile[tid] = b;
    }
    __syncthreads();
    float px = 0.0f, py = 0.0f, pz = 0.0f;
#pragma unroll 4
    for (int jj = 0; jj < width; ++jj) {
      const float4 b = tile[jj];
      pair_accel(b.x, b.y, b.z, b.w, me.x, me.y, me.z, eps2, px, py, pz);
    }
    sx += px;
    sy += py;
    sz += pz;
  }
  if (i < n) partial[(size_t)c * n + i] = make_float4(sx, sy, sz, 0.0f);
}

__global__ __launch_bounds__(256) void splitj_reduce_kernel(const float4 *__restrict__ partial,
                                                            int n, int n_chunks, float G,
                                                            float4 *__restrict__ out) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float ax = 0.0f, ay = 0.0f, az = 0.0f;
  for (int c = 0; c < n_chunks; ++c) {
    const float4 p = partial[(size_t)c * n + i];
    ax += p.x;
    ay += p.y;
    az += p.z;
  }
  out[i] = make_float4(G * ax, G * ay, G * az, 0.0f);
}

}  // namespace

size_t splitj_workspace_bytes(int64_t n, int64_t j_chunk) {
  if (n <= 0 || j_chunk < 32 || j_chunk % 32 != 0) return 0;
  const int64_t chunks = (n + j_chunk - 1) / j_chunk;
  return (size_t)chunks * (size_t)n * sizeof(float4);
}

hipError_t launch_splitj(const float *posmass, int n, float G, float eps2, float *accel,
                         int j_chunk, void *workspace, hipStream_t stream) {
  const int n_chunks = (n + j_chunk - 1) / j_chunk;
  float4 *partial = reinterpret_cast<float4 *>(workspace);
  const float4 *pm = reinterpret_cast<const float4 *>(posmass);
  const dim3 grid1((n + kSplitThreads - 1) / kSplitThreads, n_chunks);
  hipLaunchKernelGGL(splitj_partial_kernel, grid1, dim3(kSplitThreads), 0, stream, pm, n,
                     j_chunk, eps2, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(splitj_reduce_kernel, dim3((n + 255) / 256), dim3(256), 0, stream,
                     partial, n, n_chunks, G, reinterpret_cast<float4 *>(accel));
  return hipGetLastError();
}

}  // namespace nbody
