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

// Lane x receives lane x + S's value.  For S < 16 this is a DPP row_shl:S
// move inside the lane's 16-lane row (a source past the row's end reads 0);
// the tree below only uses lanes whose source lies in the same row.  S = 16
// and 32 cross rows and go through ds_bpermute.
template <int S>
__device__ __forceinline__ float lanes_down(float v) {
  if constexpr (S < 16) {
    return __int_as_float(
        __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x100 + S, 0xf, 0xf, true));
  } else {
    return __shfl_down(v, S, kWave);
  }
}

template <int S>
__device__ __forceinline__ void tree_down(float &sx, float &sy, float &sz) {
  if constexpr (S >= 1) {
    sx += lanes_down<S>(sx);
    sy += lanes_down<S>(sy);
    sz += lanes_down<S>(sz);
    tree_down<S / 2>(sx, sy, sz);
  }
}

// Tree form of the first pass (the README's section 3.2 block with the
// first-add-during-load change of its section 3.4).  A group of X lanes of a
// wavefront owns one i-body and one chunk of J = F * X j-bodies: lane x
// evaluates the F pairs j = c J + f X + x, f = 0 .. F-1, adding each term to
// its registers as it is computed, and the group then halves its width X/2,
// X/4, ..., 1 (lane x adds lane x + stride) until lane 0 holds the chunk's
// sum.  F = 1 is the plain tree; F = 2 and 4 are the page's FADL and fadl4.
// The cross-lane adds are moves within the wavefront (DPP, or ds_bpermute
// across 16-lane rows), so a tree needs no LDS storage and no barrier.  grid = (ceil(n / (256 / X)), n_chunks).
template <int X, int F>
__global__ __launch_bounds__(kSplitThreads) void splitj_tree_partial_kernel(
    const float4 *__restrict__ pm, int n, float eps2, float4 *__restrict__ partial) {
  static_assert(X >= 2 && X <= kWave && (X & (X - 1)) == 0, "tree width: power of two <= 64");
  constexpr int J = X * F;
  constexpr int IPB = kSplitThreads / X;  // i-bodies per block
  const int tid = threadIdx.x;
  const int x = tid % X;
  const int i = blockIdx.x * IPB + tid / X;
  const int c = blockIdx.y;
  const float4 me = pm[i < n ? i : n - 1];
  float sx = 0.0f, sy = 0.0f, sz = 0.0f;
#pragma unroll
  for (int f = 0; f < F; ++f) {
    const int j = c * J + f * X + x;
    const float4 b = pm[j < n ? j : n - 1];
    pair_accel(b.x, b.y, b.z, j < n ? b.w : 0.0f, me.x, me.y, me.z, eps2, sx, sy, sz);
  }
  tree_down<X / 2>(sx, sy, sz);
  if (x == 0 && i < n) partial[(size_t)c * n + i] = make_float4(sx, sy, sz, 0.0f);
}

__global__ __launch_bounds__(256) void splitj_reduce_kernel(const float4 *__restrict__ partial,
                                                            int n, int n_chunks, float G,
                                                            float4 *__restrict__ out) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float ax = 0.0f, ay = 0.0f, az = 0.0f;
  // unrolled so that several chunk rows are in flight per lane (the sum is
  // still taken in ascending chunk order)
#pragma unroll 8
  for (int c = 0; c < n_chunks; ++c) {
    const float4 p = partial[(size_t)c * n + i];
    ax += p.x;
    ay += p.y;
    az += p.z;
  }
  out[i] = make_float4(G * ax, G * ay, G * az, 0.0f);
}

template <int X, int F>
hipError_t launch_tree_partial(const float4 *pm, int n, int n_chunks, float eps2,
                               float4 *partial, hipStream_t stream) {
  constexpr int IPB = kSplitThreads / X;
  const dim3 grid((n + IPB - 1) / IPB, n_chunks);
  hipLaunchKernelGGL((splitj_tree_partial_kernel<X, F>), grid, dim3(kSplitThreads), 0, stream,
                     pm, n, eps2, partial);
  return hipGetLastError();
}

}  // namespace

bool splitj_tree_shape_ok(int64_t j_chunk, int terms) {
  if (terms != 1 && terms != 2 && terms != 4) return false;
  if (j_chunk <= 0 || j_chunk % terms != 0) return false;
  const int64_t x = j_chunk / terms;
  return x == 8 || x == 16 || x == 32 || x == 64;
}

size_t splitj_tree_workspace_bytes(int64_t n, int64_t j_chunk, int terms) {
  if (n <= 0 || !splitj_tree_shape_ok(j_chunk, terms)) return 0;
  const int64_t chunks = (n + j_chunk - 1) / j_chunk;
  return (size_t)chunks * (size_t)n * sizeof(float4);
}

hipError_t launch_splitj_tree(const float *posmass, int n, float G, float eps2, float *accel,
                              int j_chunk, int terms, void *workspace, hipStream_t stream) {
  const int n_chunks = (n + j_chunk - 1) / j_chunk;
  float4 *partial = reinterpret_cast<float4 *>(workspace);
  const float4 *pm = reinterpret_cast<const float4 *>(posmass);
  hipError_t e = hipErrorInvalidValue;
  switch (terms * 1000 + j_chunk / terms) {
#define TREE_CASE(F, X) \
  case F * 1000 + X:    \
    e = launch_tree_partial<X, F>(pm, n, n_chunks, eps2, partial, stream); \
    break;
    TREE_CASE(1, 8) TREE_CASE(1, 16) TREE_CASE(1, 32) TREE_CASE(1, 64)
    TREE_CASE(2, 8) TREE_CASE(2, 16) TREE_CASE(2, 32) TREE_CASE(2, 64)
    TREE_CASE(4, 8) TREE_CASE(4, 16) TREE_CASE(4, 32) TREE_CASE(4, 64)
#undef TREE_CASE
    default:
      return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(splitj_reduce_kernel, dim3((n + 255) / 256), dim3(256), 0, stream,
                     partial, n, n_chunks, G, reinterpret_cast<float4 *>(accel));
  return hipGetLastError();
}

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
