// Shared device helpers of libnbody (gfx950).  Internal header: not part of
// the C ABI.
//
// Arithmetic contract.  Every fused multiply-add is written out with
// __builtin_fmaf and the library is compiled with -ffp-contract=off, so the
// sequence of roundings is fixed by the source and identical in every kernel
// that uses these helpers; that is what makes the float4, float3 and SoA
// paths bitwise equal to one another.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "nbody_internal.hpp"

namespace nbody {

constexpr int kWave = 64;  // CDNA wavefront width

// One body-body term of the softened sum (README "CUDA N-Body Simulation",
// section 1.2; the 20-flop pair step of "Cuda Nbody Notes"):
//   r = x_j - x_i,  d2 = |r|^2 + eps^2,  inv = d2^{-1/2} (v_rsq_f32),
//   s = m_j inv^3,  p += s r.
// For j = i, r = 0 and the term is exactly zero (eps^2 > 0).  A padding body
// of mass 0 gives s = 0 and leaves p unchanged.
__device__ __forceinline__ void pair_accel(float xj, float yj, float zj, float mj,
                                           float xi, float yi, float zi, float eps2,
                                           float &px, float &py, float &pz) {
  const float dx = xj - xi;
  const float dy = yj - yi;
  const float dz = zj - zi;
  float d2 = __builtin_fmaf(dx, dx, eps2);
  d2 = __builtin_fmaf(dy, dy, d2);
  d2 = __builtin_fmaf(dz, dz, d2);
  const float inv = __builtin_amdgcn_rsqf(d2);
  const float s = (mj * inv) * (inv * inv);
  px = __builtin_fmaf(s, dx, px);
  py = __builtin_fmaf(s, dy, py);
  pz = __builtin_fmaf(s, dz, pz);
}

// pair_accel plus the potential sum p += mp (|r|^2 + eps^2)^{-1/2}, where the
// caller passes mp = m_j, or 0 for the j = i pair (the self term m_i / eps is
// excluded exactly: summing it and subtracting it later would cancel away
// digits whenever m_i / eps dwarfs the potential).  The acceleration
// arithmetic is the same instruction sequence as pair_accel, so (px, py, pz)
// come out bitwise equal to it.
__device__ __forceinline__ void pair_accel_pot(float xj, float yj, float zj, float mj, float mp,
                                               float xi, float yi, float zi, float eps2,
                                               float &px, float &py, float &pz, float &pp) {
  const float dx = xj - xi;
  const float dy = yj - yi;
  const float dz = zj - zi;
  float d2 = __builtin_fmaf(dx, dx, eps2);
  d2 = __builtin_fmaf(dy, dy, d2);
  d2 = __builtin_fmaf(dz, dz, d2);
  const float inv = __builtin_amdgcn_rsqf(d2);
  const float s = (mj * inv) * (inv * inv);
  px = __builtin_fmaf(s, dx, px);
  py = __builtin_fmaf(s, dy, py);
  pz = __builtin_fmaf(s, dz, pz);
  pp = __builtin_fmaf(mp, inv, pp);
}

// Lane l receives lane l - 1's value (lane 0 receives lane 63's): one step of
// the rotation that carries a j-body around the wavefront (DPP wave_ror:1).
__device__ __forceinline__ float rotate_lanes(float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x13C, 0xf, 0xf, false));
}

// Largest j with j (j + 1) / 2 <= t.
__host__ __device__ inline long long tri_root(long long t) {
  long long j = (long long)((sqrt(8.0 * (double)t + 1.0) - 1.0) * 0.5);
  while (j > 0 && j * (j + 1) / 2 > t) --j;
  while ((j + 1) * (j + 2) / 2 <= t) ++j;
  return j;
}

// Order of the P (P + 1) / 2 panel pairs (I, J), I <= J < P, of the
// pair-symmetric passes, and which blocks take them.
//
// Pairs are numbered in tile-column order: the panels are grouped in tiles
// of S x S panel pairs; tile column c holds the pairs with
// J in [cS, cS + cols), cols = min(S, P - cS), which are the pairs numbered
// from Sc (Sc + 1) / 2 on (exactly as in the plain J-major triangle).  Inside
// a tile column come the full tiles of rows a = 0 .. c - 1 (S x cols pairs
// each, J-major), then the triangle of the diagonal tile.  A stretch of
// consecutive numbers therefore touches about S + stretch / S panels.
//
// A launch may take a contiguous range of the numbers, [t0, t0 + pairs): a
// range of whole tile columns is the set of pairs with J in a range of
// panels, which is how the pair-symmetric pass is cut into column chunks.
//
// Blocks go to the 8 XCDs of the chip round robin (block b to XCD b % 8), so
// block b takes pair number t0 + (b % 8) * per_xcd + b / 8: each XCD walks
// its own contiguous stretch of the order, and the panels its concurrent
// blocks read stay in that XCD's L2.  Which block computes a pair does not
// change any sum: every pair writes its own workspace slot.
struct PanelOrder {
  int P;               // panels
  int S;               // tile side in panels
  long long t0;        // number of the launch's first pair
  long long pairs;     // pairs in the launch (P (P + 1) / 2 for all of them)
  long long per_xcd;   // ceil(pairs / 8): grid = 8 * per_xcd blocks
};

constexpr int kXcds = 8;
constexpr int kPanelTile = 32;

// The pairs numbered [t0, t1) of P panels.
inline PanelOrder panel_order_range(long long P, long long t0, long long t1) {
  PanelOrder o;
  o.P = (int)P;
  o.S = kPanelTile;
  o.t0 = t0;
  o.pairs = t1 - t0;
  o.per_xcd = (o.pairs + kXcds - 1) / kXcds;
  return o;
}

// Every pair of P panels.
inline PanelOrder panel_order(long long P) { return panel_order_range(P, 0, P * (P + 1) / 2); }

// The pairs numbered [first, last) of P panels, one block of `threads`
// threads per pair, in as few launches as launch_block_cap allows:
// launch(order, blocks) issues one of them.  A block finds its pair from the
// order alone, so the split leaves every pair's work unchanged.  Returns the
// first launch error.
template <class F>
hipError_t launch_pair_ranges(long long P, long long first, long long last, int threads,
                              F launch) {
  long long cap = launch_block_cap(threads) / kXcds * kXcds;
  if (cap < kXcds) cap = kXcds;
  for (long long t0 = first; t0 < last; t0 += cap) {
    const PanelOrder o = panel_order_range(P, t0, t0 + cap < last ? t0 + cap : last);
    launch(o, kXcds * o.per_xcd);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Number of the first pair with J >= c (c a multiple of the tile side, or P).
__host__ __device__ inline long long first_pair_of_column(long long c) { return c * (c + 1) / 2; }

// Pair number t (0 <= t < pairs) of the order above.
__host__ __device__ inline void panel_pair_of(const PanelOrder &o, long long t, int &I, int &J) {
  const long long S = o.S;
  const long long c = tri_root(t) / S;             // tile column of t
  const long long u = t - (S * c) * (S * c + 1) / 2;  // offset inside the tile column
  const long long cols = (o.P - S * c) < S ? (o.P - S * c) : S;
  if (u < c * S * cols) {                          // full tile of row a, J-major
    const long long a = u / (S * cols), v = u % (S * cols);
    J = (int)(S * c + v / S);
    I = (int)(S * a + v % S);
  } else {                                         // diagonal tile, I <= J
    const long long v = u - c * S * cols;
    const long long j = tri_root(v);
    J = (int)(S * c + j);
    I = (int)(S * c + v - j * (j + 1) / 2);
  }
}

// The pair block b takes; false for the few blocks past the launch's last
// pair.
__host__ __device__ inline bool panel_pair_of_block(const PanelOrder &o, long long b, int &I,
                                                    int &J, long long &t) {
  const long long k = b / kXcds;
  const long long u = (b % kXcds) * o.per_xcd + k;
  if (k >= o.per_xcd || u >= o.pairs) return false;
  t = o.t0 + u;
  panel_pair_of(o, t, I, J);
  return true;
}

// Where the pair-symmetric pass keeps panel K's sums from panel J, for a
// launch that takes the panel pairs (I, J') with J' in [c0, c1) (a column
// chunk; the whole pass is the chunk [0, P)):
//  - a panel K < c0 gets one slot per column of the chunk (its i-side sums
//    from panels c0 .. c1 - 1): slot K (c1 - c0) + (J - c0);
//  - a panel K in [c0, c1) gets its sums from every panel J < c1 (j-side
//    from the panels before it, its own diagonal pair, i-side from the
//    chunk's later panels): slot c0 (c1 - c0) + (K - c0) c1 + J.
// For either kind of panel, consecutive J have consecutive slots.  A panel
// K >= c1 gets nothing from the chunk.  The whole pass ([0, P)) is slot
// K P + J.
struct SlotMap {
  int c0, c1;
  __host__ __device__ long long slot(int K, int J) const {
    const long long w = c1 - c0;
    return K < c0 ? (long long)K * w + (J - c0)
                  : (long long)c0 * w + (long long)(K - c0) * c1 + J;
  }
  __host__ __device__ long long slots() const { return (long long)(c1 - c0) * (c0 + c1); }
};

// ---------------------------------------------------------------------------
// Body loaders / storers for the three layouts.  load(j) returns (x, y, z, m);
// the caller clamps j into [0, n) and zeroes m for padding.
// ---------------------------------------------------------------------------
struct LayoutAos4 {
  const float4 *pm;
  float4 *out;
  __device__ __forceinline__ float4 load(int j) const { return pm[j]; }
  __device__ __forceinline__ void store(int i, float ax, float ay, float az) const {
    out[i] = make_float4(ax, ay, az, 0.0f);
  }
  __device__ __forceinline__ void store4(int i, float ax, float ay, float az, float w) const {
    out[i] = make_float4(ax, ay, az, w);
  }
};

struct LayoutAos3 {
  const float *pos;   // [n][3]
  const float *mass;  // [n]
  float *out;         // [n][3]
  __device__ __forceinline__ float4 load(int j) const {
    const size_t b = (size_t)j * 3;
    return make_float4(pos[b], pos[b + 1], pos[b + 2], mass[j]);
  }
  __device__ __forceinline__ void store(int i, float ax, float ay, float az) const {
    const size_t b = (size_t)i * 3;
    out[b] = ax;
    out[b + 1] = ay;
    out[b + 2] = az;
  }
};

struct LayoutSoa {
  const float *x, *y, *z, *m;
  float *ax, *ay, *az;
  __device__ __forceinline__ float4 load(int j) const {
    return make_float4(x[j], y[j], z[j], m[j]);
  }
  __device__ __forceinline__ void store(int i, float vx, float vy, float vz) const {
    ax[i] = vx;
    ay[i] = vy;
    az[i] = vz;
  }
};

}  // namespace nbody
