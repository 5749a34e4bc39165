// Pair-symmetric force pass: every unordered pair of bodies is evaluated
// once and its term goes to both bodies (Newton's third law: the term on j
// from i is the term on i from j times -m_i/m_j).  The atomics tutorial (CUDA
// programming part 9, its neighbour-list example) runs the same symmetric
// half loop but has to add the second body's share with atomicAdd.  Here the
// share is carried by the j-body's own state and added in a fixed order, so
// the result is bitwise reproducible and there are no atomics.
//
// Decomposition.  Bodies are cut into P panels of B = 64 * W * K bodies (the
// tail padded with zero-mass copies of the last body).  A block takes one
// task (I, J), I <= J, of the P(P+1)/2 panel pairs (in the XCD-aware tile
// order of PanelOrder, which keeps each XCD's panels in its own L2):
//  - wave w holds K bodies of panel I per lane in registers (its i-group);
//  - panel J is walked in sweeps of 64 * KP bodies.  Over the 64 steps of a
//    sweep every lane meets every j-body of the sweep once, evaluating its
//    K x KP pairs per step;
//  - pair term: r = x_j - x_i, inv = rsq(|r|^2 + eps^2), w = inv^3;
//    i gains m_j w r (register sum), j gains -m_i w r (the j-side sum);
//  - the W waves' j-side sums are added in ascending wave order through LDS.
// The j-state (x, y, z, m and the j-side sums) travels in one of two ways:
//  - rotated (JL = 0): each lane loads KP j-bodies and after each step moves
//    the j-state one lane along the wave with a DPP wave_ror:1 move (7 / K
//    moves per pair, VALU instructions that cannot dual-issue);
//  - LDS-carried (JL > 0, KP = 1): the j-bodies and their sums sit in the
//    wave's LDS; each step a lane reads the body it meets, sums its K pairs'
//    j-side terms in registers, then adds them to the body's slot (a read, 3
//    adds and a write: the adds dual-issue, and no DPP moves are left).
// Diagonal tasks (I = J) of the 4-wave variants use the one-sided sum (j
// over the whole panel, self term exactly 0) and no j-side sums; those of the
// one-wave variants are pair-symmetric within the panel (sym_diag_task), each
// pair once in the one-sided pass's mass-first form, at about half the
// cost.
//
// Output of a task: panel I's sums from panel J and, for I < J, panel J's
// sums from panel I, each in its own workspace slot of NC x B floats (NC = 3
// sums per body, 4 with the potential).  A second kernel forms
// a_i = G * sum_{J = 0 .. P-1} part[I(i)][J][i], the J in blocks of 32
// panels (ascending within a block, block sums ascending).
// The pass runs either whole (one task launch over all P (P + 1) / 2 panel
// pairs, slots [P][P]: 12 N^2 / B bytes) or in column chunks: a launch takes
// the pairs with J in [c0, c1) (SlotMap gives their slots; c0 and c1 are
// multiples of 32, or c1 = P), and the chunk's reduce continues each touched
// body's fp32 running sum (kept in accel_out between chunks) with that
// chunk's blocks.  A body's panel sums are then added in the same order as in
// the whole pass, so the two give bitwise equal results; the chunked
// workspace is two chunks' slots (consecutive chunks overlap on two queues),
// about 48 N C bytes for chunks of C panels.
//
// Per pair (two interactions) a lane issues 16 FP32 VALU ops and one
// v_rsq_f32, plus 7 / K DPP moves (rotated) or 3 / K adds (LDS-carried); the
// one-sided kernel issues 12 ops and one v_rsq_f32 per interaction.
#include "nbody_common.hpp"
#include "nbody_internal.hpp"

#include <algorithm>
#include <mutex>
#include <vector>

namespace nbody {

namespace {

// One step of the off-diagonal sweep: the lane's K i-bodies against its
// current j-body.  The pairs are processed IL at a time in phases (all
// differences, then all d^2, all rsq, ...), which gives each wave IL
// independent chains to issue from; IL = 1 is one pair after the other.  The
// arithmetic of each pair, and its order of accumulation, do not depend on IL.
// POT adds the potential sums: i gains m_j inv, j gains m_i inv (two more
// multiply-adds per pair; the force arithmetic is unchanged).  The last ML of
// the K i-masses are read from LDS (mil[r * 64], r = 0 .. ML - 1) instead of
// registers.  FRESH starts the j-side sums at this step: the first pair's
// term is stored, not added.
template <int K, int IL, bool POT, int ML, bool FRESH = false>
__device__ __forceinline__ void sym_step(const float (&xi)[K], const float (&yi)[K],
                                         const float (&zi)[K], const float (&mi)[K],
                                         const float *mil, float xj,
                                         float yj, float zj, float mj, float eps2, float (&ax)[K],
                                         float (&ay)[K], float (&az)[K], float (&ap)[K],
                                         float &cx, float &cy, float &cz, float &cp) {
  static_assert(K % IL == 0, "interleave width must divide K");
#pragma unroll
  for (int h = 0; h < K; h += IL) {
    float dx[IL], dy[IL], dz[IL], inv[IL], w[IL];
#pragma unroll
    for (int q = 0; q < IL; ++q) {
      dx[q] = xj - xi[h + q];
      dy[q] = yj - yi[h + q];
      dz[q] = zj - zi[h + q];
    }
#pragma unroll
    for (int q = 0; q < IL; ++q) w[q] = __builtin_fmaf(dx[q], dx[q], eps2);
#pragma unroll
    for (int q = 0; q < IL; ++q) w[q] = __builtin_fmaf(dy[q], dy[q], w[q]);
#pragma unroll
    for (int q = 0; q < IL; ++q) w[q] = __builtin_fmaf(dz[q], dz[q], w[q]);
#pragma unroll
    for (int q = 0; q < IL; ++q) inv[q] = __builtin_amdgcn_rsqf(w[q]);
#pragma unroll
    for (int q = 0; q < IL; ++q) w[q] = (inv[q] * inv[q]) * inv[q];
#pragma unroll
    for (int q = 0; q < IL; ++q) {
      const float sj = mj * w[q];
      ax[h + q] = __builtin_fmaf(sj, dx[q], ax[h + q]);
      ay[h + q] = __builtin_fmaf(sj, dy[q], ay[h + q]);
      az[h + q] = __builtin_fmaf(sj, dz[q], az[h + q]);
      if constexpr (POT) ap[h + q] = __builtin_fmaf(mj, inv[q], ap[h + q]);
    }
#pragma unroll
    for (int q = 0; q < IL; ++q) {
      const float m = (h + q >= K - ML) ? mil[(h + q - (K - ML)) * kWave] : mi[h + q];
      const float si = m * w[q];
      if (FRESH && h + q == 0) {  // the j-side sums start at this step
        cx = si * dx[q];
        cy = si * dy[q];
        cz = si * dz[q];
        if constexpr (POT) cp = m * inv[q];
      } else {
        cx = __builtin_fmaf(si, dx[q], cx);
        cy = __builtin_fmaf(si, dy[q], cy);
        cz = __builtin_fmaf(si, dz[q], cz);
        if constexpr (POT) cp = __builtin_fmaf(m, inv[q], cp);
      }
    }
  }
}

// This lane's index in the wavefront, computed afresh where it is used: an
// asm the compiler can neither merge with an earlier one nor hoist, so that
// no lane index (or address made from one) has to be kept in a register, or
// spilled, across the step loop of a sweep.
__device__ __forceinline__ int fresh_lane() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// A wave's issue priority from how far it has come: 3 in the first quarter
// of its steps, down to 0 in the last (quarter is wave-uniform).  The SIMD
// issues from the highest priority first, so waves that are behind catch up.
__device__ __forceinline__ void pace(int quarter) {
  if (quarter <= 0)
    __builtin_amdgcn_s_setprio(3);
  else if (quarter == 1)
    __builtin_amdgcn_s_setprio(2);
  else if (quarter == 2)
    __builtin_amdgcn_s_setprio(1);
  else
    __builtin_amdgcn_s_setprio(0);
}

// Sums kept per body: the three acceleration components, plus the potential
// sum with POT.
template <bool POT>
constexpr int sym_sums() {
  return POT ? 4 : 3;
}

template <int K, int KP, int W, int IL, bool POT, int ML, int JL, bool DIAG>
__device__ __forceinline__ void sym_task(const float4 *__restrict__ pm, int n, int I, int J,
                                         SlotMap map, float eps2, float *__restrict__ part,
                                         float (*csum)[KP][sym_sums<POT>()][kWave], float *mis,
                                         float4 *jtile, float4 *jsum) {
  constexpr int B = W * kWave * K;
  constexpr int JG = kWave * KP;
  constexpr int NG = B / JG;
  constexpr int NC = sym_sums<POT>();
  const int tid = (int)threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  // The task's two slots: panel I's sums from J, panel J's sums from I.  For
  // 8 i-bodies per lane their addresses are formed once per task, for fewer
  // at each use.  The addresses are the same either way; the forms differ in
  // what the compiler keeps live across the step loop, and with it where it
  // places each step's slot read: these are the faster forms, measured on
  // MI355X (2^20 bodies, K = 8: 185.0 against 187.7 ms; 131072 bodies,
  // K = 4: 3.06 against 3.13 ms).
  constexpr bool kHoist = K >= 8;
  constexpr bool kPace = W == 1;
  float *const part_ij = part + (size_t)map.slot(I, J) * NC * B;
  float *const part_ji = part + (size_t)map.slot(J, I) * NC * B;

  float xi[K], yi[K], zi[K], mi[K], ax[K], ay[K], az[K], ap[K];
#pragma unroll
  for (int q = 0; q < K; ++q) {
    const int i = I * B + wave * (kWave * K) + q * kWave + lane;
    const float4 b = pm[i < n ? i : n - 1];
    xi[q] = b.x;
    yi[q] = b.y;
    zi[q] = b.z;
    mi[q] = i < n ? b.w : 0.0f;
    if constexpr (ML > 0) {
      if (q >= K - ML) mis[(wave * ML + q - (K - ML)) * kWave + lane] = mi[q];
    }
    ax[q] = 0.0f;
    ay[q] = 0.0f;
    az[q] = 0.0f;
    ap[q] = 0.0f;
  }

  if constexpr (JL > 0 && !DIAG) {
    // The j-state lives in the wave's LDS instead of travelling along the
    // lanes.  The sweep's 64 j-bodies sit twice in a row in the tile jt, and
    // step s pairs lane l with entry k = l + s, i.e. body (l + s) mod 64.  The
    // j-side sums sit in slots js[k] beside them: the lane reads slot k, adds
    // its K pairs' terms in registers and writes the slot back.  The next
    // access to slot k is lane l - 1's at step s + 1, an instruction the LDS
    // executes after this write (one wave's LDS instructions run in issue
    // order).  Body j's sum of the sweep is js[j] + js[j + 64].
    static_assert(KP == 1, "LDS j-tiles hold one j-body per lane");
    constexpr int U = JL;  // steps per unrolled block: LDS offsets are immediates
    static_assert(kWave % U == 0, "unroll must divide the sweep");
    float4 *jt = jtile + wave * 2 * kWave;
    float4 *js = jsum + wave * 2 * kWave;
    // byte offset of the lane's first LDS mass; the empty asm that claims to
    // change it every step keeps the mass reads inside the step (it is the
    // same register in and out, so it costs no instruction)
    int mio = (wave * ML * kWave + lane) * (int)sizeof(float);
    for (int g = 0; g < NG; ++g) {
      const int j = J * B + g * kWave + lane;
      const float4 b = pm[j < n ? j : n - 1];
      const float4 jb = make_float4(b.x, b.y, b.z, j < n ? b.w : 0.0f);
      jt[lane] = jb;
      jt[lane + kWave] = jb;
      // a zero made here, so that the compiler has no zero vector to keep
      // (or spill) across the sweep
      float z;
      asm volatile("v_mov_b32 %0, 0" : "=v"(z));
      js[lane] = make_float4(z, z, z, z);
      js[lane + kWave] = make_float4(z, z, z, z);
      // Other lanes read what this lane wrote: no LDS access may be moved
      // across these points (the empty asm with a memory clobber).
      asm volatile("" ::: "memory");
      float4 y = jt[lane];
      // paced tasks take the sweep in two halves, each at its own priority
      constexpr int kHalves = kPace ? 2 : 1;
      for (int h = 0; h < kHalves; ++h) {
      if constexpr (kPace) pace((2 * (2 * g + h)) / NG);
      for (int s0 = h * (kWave / kHalves); s0 < (h + 1) * (kWave / kHalves); s0 += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int k = lane + s0 + u;
          const float4 yn = jt[k + 1];  // the next step's j-body (k + 1 <= 127)
          if constexpr (ML > 0) asm volatile("" : "+v"(mio));
          const float *mil =
              reinterpret_cast<const float *>(reinterpret_cast<const char *>(mis) + mio);
          float tx, ty, tz, tp;
          sym_step<K, IL, POT, ML, true>(xi, yi, zi, mi, mil, y.x, y.y, y.z, y.w, eps2, ax, ay,
                                         az, ap, tx, ty, tz, tp);
          // the slot is read after the step's pairs: its last writer is the
          // neighbour lane's previous step, already behind this point
          float4 c = js[k];
          c.x += tx;
          c.y += ty;
          c.z += tz;
          if constexpr (POT) c.w += tp;
          js[k] = c;
          asm volatile("" ::: "memory");
          y = yn;
        }
      }
      }
      // j-side sums of this sweep: add the W waves in ascending order
      // W waves add each other's sums: a block barrier; a one-wave task reads
      // only its own lanes' slots, which one wave's LDS instructions order
      if constexpr (W > 1)
        __syncthreads();
      else
        asm volatile("" ::: "memory");
      for (int e = tid; e < NC * kWave; e += W * kWave) {
        const int c = e / kWave, l = e % kWave;
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < W; ++w) {
          const float *sw = reinterpret_cast<const float *>(jsum + w * 2 * kWave);
          sum += sw[4 * l + c] + sw[4 * (l + kWave) + c];
        }
        // the force on j from i points the other way; the potential does not
        if constexpr (kHoist)
          part_ji[(size_t)c * B + g * kWave + l] = c < 3 ? -sum : sum;
        else
          part[((size_t)map.slot(J, I) * NC + c) * B + g * kWave + l] = c < 3 ? -sum : sum;
      }
      if constexpr (W > 1)
        __syncthreads();
      else
        asm volatile("" ::: "memory");
    }
  } else {
    for (int g = 0; g < NG; ++g) {
      if constexpr (kPace) pace((4 * g) / NG);
      float xj[KP], yj[KP], zj[KP], mj[KP], cx[KP], cy[KP], cz[KP], cp[KP];
#pragma unroll
      for (int p = 0; p < KP; ++p) {
        const int j = J * B + g * JG + p * kWave + lane;
        const float4 b = pm[j < n ? j : n - 1];
        xj[p] = b.x;
        yj[p] = b.y;
        zj[p] = b.z;
        mj[p] = j < n ? b.w : 0.0f;
        cx[p] = 0.0f;
        cy[p] = 0.0f;
        cz[p] = 0.0f;
        cp[p] = 0.0f;
      }
      for (int s = 0; s < kWave; ++s) {
#pragma unroll
        for (int p = 0; p < KP; ++p) {
          if constexpr (!DIAG) {
            // masses kept in LDS are read inside the step: the empty asm that
            // claims to change the index stops the compiler from hoisting the
            // reads out of the loop into registers
            int mio = wave * ML * kWave + lane;
            if constexpr (ML > 0) asm volatile("" : "+v"(mio));
            sym_step<K, IL, POT, ML>(xi, yi, zi, mi, mis + mio, xj[p], yj[p], zj[p], mj[p], eps2,
                                     ax, ay, az, ap, cx[p], cy[p], cz[p], cp[p]);
          } else {
#pragma unroll
            for (int q = 0; q < K; ++q) {
              const float dx = xj[p] - xi[q];
              const float dy = yj[p] - yi[q];
              const float dz = zj[p] - zi[q];
              float d2 = __builtin_fmaf(dx, dx, eps2);
              d2 = __builtin_fmaf(dy, dy, d2);
              d2 = __builtin_fmaf(dz, dz, d2);
              const float inv = __builtin_amdgcn_rsqf(d2);
              const float sj = (mj[p] * inv) * (inv * inv);
              ax[q] = __builtin_fmaf(sj, dx, ax[q]);
              ay[q] = __builtin_fmaf(sj, dy, ay[q]);
              az[q] = __builtin_fmaf(sj, dz, az[q]);
              if constexpr (POT) {
                // lane l meets its own body at step 0 of the sweep whose j-bodies
                // are that body's group: the self term m_i / eps is left out
                const bool self = s == 0 && g * KP + p == wave * K + q;
                ap[q] = __builtin_fmaf(self ? 0.0f : mj[p], inv, ap[q]);
              }
            }
          }
          xj[p] = rotate_lanes(xj[p]);
          yj[p] = rotate_lanes(yj[p]);
          zj[p] = rotate_lanes(zj[p]);
          mj[p] = rotate_lanes(mj[p]);
          if constexpr (!DIAG) {
            cx[p] = rotate_lanes(cx[p]);
            cy[p] = rotate_lanes(cy[p]);
            cz[p] = rotate_lanes(cz[p]);
            if constexpr (POT) cp[p] = rotate_lanes(cp[p]);
          }
        }
      }
      if constexpr (!DIAG) {
        // j-side sums of this sweep: add the W waves in ascending order
#pragma unroll
        for (int p = 0; p < KP; ++p) {
          csum[wave][p][0][lane] = cx[p];
          csum[wave][p][1][lane] = cy[p];
          csum[wave][p][2][lane] = cz[p];
          if constexpr (POT) csum[wave][p][3][lane] = cp[p];
        }
        __syncthreads();
        for (int e = tid; e < KP * NC * kWave; e += W * kWave) {
          const int p = e / (NC * kWave), c = (e / kWave) % NC, l = e % kWave;
          float sum = 0.0f;
#pragma unroll
          for (int w = 0; w < W; ++w) sum += csum[w][p][c][l];
          // the force on j from i points the other way; the potential does not
          part[((size_t)map.slot(J, I) * NC + c) * B + g * JG + p * kWave + l] = c < 3 ? -sum : sum;
        }
        __syncthreads();
      }
    }
  }

  if constexpr (kHoist) {
    const int lo = fresh_lane();
#pragma unroll
    for (int q = 0; q < K; ++q) {
      float *row = part_ij + wave * (kWave * K) + q * kWave;
      row[lo] = ax[q];
      row[B + lo] = ay[q];
      row[2 * B + lo] = az[q];
      if constexpr (POT) row[3 * B + lo] = ap[q];
    }
  } else {
#pragma unroll
    for (int q = 0; q < K; ++q) {
      const int b = wave * (kWave * K) + q * kWave + lane;
      float *row = part + (size_t)map.slot(I, J) * NC * B + b;
      row[0] = ax[q];
      row[B] = ay[q];
      row[2 * B] = az[q];
      if constexpr (POT) row[3 * B] = ap[q];
    }
  }
}

// A diagonal panel pair (I, I) of a one-wave task, each unordered pair of the
// panel met once (the off-diagonal sweep would meet every pair twice).  The
// panel's j-groups g (64 bodies each) are taken from the last to the first;
// group g is staged twice in a row in the wave's LDS tile with zeroed slots,
// as in the off-diagonal sweep.  The lane's i-bodies of the groups q < g meet
// all 64 j-bodies (steps 0 .. 63), and its i-body of group g meets the
// bodies 1 .. 32 lanes ahead (at 32 only lanes 0 .. 31, so that each pair of
// the group is met once and no body meets itself).  i-side terms gather in
// registers, j-side terms in the group's LDS slots under the same in-order
// rule as the off-diagonal sweep.  After group g both sums of its bodies are
// complete (later groups are earlier ones, which meet g only as j-bodies), so
// its panel sums are written then: i-side minus j-side (the potential: plus).
// About half the work of an off-diagonal task.
template <int K, bool POT>
__device__ __forceinline__ void sym_diag_task(const float4 *__restrict__ pm, int n, int I,
                                              SlotMap map, float eps2, float *__restrict__ part,
                                              float4 *jt, float4 *js) {
  constexpr int B = kWave * K;
  constexpr int NC = sym_sums<POT>();
  const int lane = (int)threadIdx.x % kWave;
  float xi[K], yi[K], zi[K], mi[K], ax[K], ay[K], az[K], ap[K];
#pragma unroll
  for (int q = 0; q < K; ++q) {
    const int i = I * B + q * kWave + lane;
    const float4 b = pm[i < n ? i : n - 1];
    xi[q] = b.x;
    yi[q] = b.y;
    zi[q] = b.z;
    mi[q] = i < n ? b.w : 0.0f;
    ax[q] = 0.0f;
    ay[q] = 0.0f;
    az[q] = 0.0f;
    ap[q] = 0.0f;
  }
  // one pair: this lane's i-body q and the j-body in tile entry k, the j-side
  // term added into slot k (q is a constant once the loops are unrolled)
  auto pair = [&](int q, int k) {
    const float4 y = jt[k];
    const float dx = y.x - xi[q];
    const float dy = y.y - yi[q];
    const float dz = y.z - zi[q];
    float w = __builtin_fmaf(dx, dx, eps2);
    w = __builtin_fmaf(dy, dy, w);
    w = __builtin_fmaf(dz, dz, w);
    const float inv = __builtin_amdgcn_rsqf(w);
    const float inv2 = inv * inv;
    // mass first, as in the one-sided pass: the zero-mass copies of body n - 1
    // that pad the last panel sit on that body, and a zero mass must turn
    // their terms into exact zeros for any eps2 > 0
    const float sj = (y.w * inv) * inv2;
    ax[q] = __builtin_fmaf(sj, dx, ax[q]);
    ay[q] = __builtin_fmaf(sj, dy, ay[q]);
    az[q] = __builtin_fmaf(sj, dz, az[q]);
    if constexpr (POT) ap[q] = __builtin_fmaf(y.w, inv, ap[q]);
    const float si = (mi[q] * inv) * inv2;
    float4 c = js[k];
    c.x = __builtin_fmaf(si, dx, c.x);
    c.y = __builtin_fmaf(si, dy, c.y);
    c.z = __builtin_fmaf(si, dz, c.z);
    if constexpr (POT) c.w = __builtin_fmaf(mi[q], inv, c.w);
    js[k] = c;
    // the slot's next access is another lane's, one pair later
    asm volatile("" ::: "memory");
  };
  float *row = part + (size_t)map.slot(I, I) * NC * B;
#pragma unroll
  for (int g = K - 1; g >= 0; --g) {
    const int j = I * B + g * kWave + lane;
    const float4 b = pm[j < n ? j : n - 1];
    const float4 jb = make_float4(b.x, b.y, b.z, j < n ? b.w : 0.0f);
    jt[lane] = jb;
    jt[lane + kWave] = jb;
    js[lane] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    js[lane + kWave] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    asm volatile("" ::: "memory");
#pragma unroll
    for (int q = 0; q < g; ++q) {
#pragma unroll 8
      for (int s = 0; s < kWave; ++s) pair(q, lane + s);
    }
#pragma unroll 8
    for (int s = 1; s < kWave / 2; ++s) pair(g, lane + s);
    if (lane < kWave / 2) pair(g, lane + kWave / 2);
    asm volatile("" ::: "memory");
    // group g's panel sums; a lane reads only its own bodies' slots
    const float4 lo = js[lane], hi = js[lane + kWave];
    const int bg = g * kWave + lane;
    row[bg] = ax[g] - (lo.x + hi.x);
    row[B + bg] = ay[g] - (lo.y + hi.y);
    row[2 * B + bg] = az[g] - (lo.z + hi.z);
    if constexpr (POT) row[3 * B + bg] = ap[g] + (lo.w + hi.w);
    // the next group overwrites the tile after every lane's reads
    asm volatile("" ::: "memory");
  }
}

// One task (panel pair) per block of W waves.  PanelOrder gives the pair of
// each block: every XCD walks a contiguous stretch of tile-ordered pairs.
template <int K, int KP, int W, int OCC, int IL, bool POT, int ML, int JL>
__global__ __launch_bounds__(W *kWave) __attribute__((amdgpu_waves_per_eu(OCC))) void
symmetric_task_kernel(const float4 *__restrict__ pm, int n, PanelOrder order, SlotMap map,
                      float eps2, float *__restrict__ part) {
  constexpr int NC = sym_sums<POT>();
  // one-wave tasks are paced (see pace): a wave starts at the top priority
  if constexpr (W == 1) __builtin_amdgcn_s_setprio(3);
  __shared__ float csum[JL > 0 ? 1 : W][KP][NC][kWave];
  __shared__ float mis[ML > 0 ? W * ML * kWave : 1];
  __shared__ float4 jtile[JL > 0 ? W * 2 * kWave : 1];
  __shared__ float4 jsum[JL > 0 ? W * 2 * kWave : 1];
  int Ic, Jc;
  long long t;
  // the block returns as a whole, so no barrier is skipped
  if (!panel_pair_of_block(order, blockIdx.x, Ic, Jc, t)) return;
  Ic = __builtin_amdgcn_readfirstlane(Ic);
  Jc = __builtin_amdgcn_readfirstlane(Jc);
  if (Ic == Jc) {
    if constexpr (W == 1 && JL > 0)
      sym_diag_task<K, POT>(pm, n, Ic, map, eps2, part, jtile, jsum);
    else
      sym_task<K, KP, W, IL, POT, ML, JL, true>(pm, n, Ic, Jc, map, eps2, part, csum, mis, jtile,
                                                jsum);
  } else
    sym_task<K, KP, W, IL, POT, ML, JL, false>(pm, n, Ic, Jc, map, eps2, part, csum, mis, jtile,
                                               jsum);
}

// The panel sums of one launch's slots (SlotMap map, columns [c0, c1)) added
// into each touched body's sum in ascending J, in two levels: the slots of
// each block of 32 consecutive panels (J in [32 k, 32 k + 32)) are added in
// order into a fresh block sum, and the block sums are added in order into
// the body's sum.  A body of a panel K < c0 continues the fp32 running sum an
// earlier chunk left in out[i] with the blocks of J = c0 .. c1 - 1; a body of
// a panel in [c0, c1) starts from 0 with the blocks of J = 0 .. c1 - 1.
// Chunk bounds are multiples of 32 (or P), so a chunked pass forms the same
// blocks, in the same order, as the whole pass.  The last chunk (c1 = P)
// writes a_i = G * sum (with POT the fourth sum is phi_i and w = Phi_i =
// -G phi_i, else w = 0); earlier chunks write the unscaled running sums.  The
// bodies of panels K >= c1 are not touched: the caller launches the bodies
// below min(n, c1 B).
//
// A block of 4 waves takes 64 bodies (one panel: B is a multiple of 64) and
// one component (blockIdx.y); its waves form 4 block sums at a time and
// wave 0 adds them in order.  That gives small n several waves per SIMD
// where one thread per body walking all P slots would not.
constexpr int kReduceWaves = 4;

template <bool POT>
__global__ __launch_bounds__(kReduceWaves *kWave) void symmetric_reduce_kernel(
    const float *__restrict__ part, int n, int B, SlotMap map, int last, float G,
    float4 *__restrict__ out) {
  constexpr int NC = sym_sums<POT>();
  constexpr int JB = kPanelTile;  // panels per block sum
  __shared__ float blk[kReduceWaves][kWave];
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
  const int lane = (int)threadIdx.x % kWave;
  const int i0 = blockIdx.x * kWave;
  const int i = i0 + lane;
  const int c = blockIdx.y;
  const bool live = i < n;
  const int K = i0 / B;  // the same panel for the 64 bodies
  const int b = i % B;
  float *o = reinterpret_cast<float *>(out) + (size_t)i * 4;
  const int J0 = K < map.c0 ? map.c0 : 0, J1 = map.c1;
  float sum = 0.0f;
  if (K < map.c0 && live && wave == 0) sum = o[c];
  const int nb = (J1 - J0 + JB - 1) / JB;
  for (int r = 0; r < nb; r += kReduceWaves) {
    const int jb = r + wave;
    float p = 0.0f;
    if (jb < nb && live) {
      const int ja = J0 + jb * JB, je = min(J1, ja + JB);
      const float *s = part + ((size_t)map.slot(K, ja) * NC + c) * B + b;
#pragma unroll 8
      for (int J = ja; J < je; ++J, s += (size_t)NC * B) p += s[0];
    }
    blk[wave][lane] = p;
    __syncthreads();
    if (wave == 0) {
      for (int w = 0; w < kReduceWaves && r + w < nb; ++w) sum += blk[w][lane];
    }
    __syncthreads();
  }
  if (wave == 0 && live) {
    // the fourth sum (with the potential) is phi_i, stored as Phi_i = -G phi_i;
    // without it, w is 0
    o[c] = last ? (c < 3 ? G * sum : -G * sum) : sum;
    if (!POT && c == 0) o[3] = 0.0f;
  }
}

// The same sums with one thread per (body, component) and 256 consecutive
// bodies per block, each thread walking all of its body's blocks of 32 panels
// in turn: the same block sums, added in the same order, so the results are
// bitwise those of symmetric_reduce_kernel.  Launches over many bodies use it:
// a block's four waves then read 1 KB of consecutive bodies from each slot,
// where the split form reads 256-byte runs from four slots far apart.
template <bool POT>
__global__ __launch_bounds__(256) void symmetric_reduce_walk_kernel(
    const float *__restrict__ part, int n, int B, SlotMap map, int last, float G,
    float4 *__restrict__ out) {
  constexpr int NC = sym_sums<POT>();
  constexpr int JB = kPanelTile;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int c = blockIdx.y;
  const int K = i / B;
  float *o = reinterpret_cast<float *>(out) + (size_t)i * 4;
  const int J0 = K < map.c0 ? map.c0 : 0, J1 = map.c1;
  float sum = K < map.c0 ? o[c] : 0.0f;
  // a panel's slots for consecutive J are consecutive
  const float *s = part + ((size_t)map.slot(K, J0) * NC + c) * B + i % B;
  for (int ja = J0; ja < J1; ja += JB) {
    const int je = min(J1, ja + JB);
    float p = 0.0f;
#pragma unroll 8
    for (int J = ja; J < je; ++J, s += (size_t)NC * B) p += s[0];
    sum += p;
  }
  o[c] = last ? (c < 3 ? G * sum : -G * sum) : sum;
  if (!POT && c == 0) o[3] = 0.0f;
}

// (id, K, KP, waves, occupancy target, interleave width, i-masses in LDS,
// JL: 0 = rotated j-state, else LDS-carried with JL steps per unrolled
// block); panel B = 64 * waves * K.  Ids are part of the ABI
// (nbody_accel_symmetric):
//  0  8 i-bodies per lane in 4-wave blocks (2048-body panels), five of the
//     eight i-masses in LDS so that the kernel fits 72 VGPRs (7 waves per
//     SIMD): the library's choice above 3e5 bodies;
//  1  4 i-bodies per lane in 4-wave blocks (1024-body panels, 8 waves per
//     SIMD): from 77824 to 3e5 bodies;
//  2  4 i-bodies per lane in one-wave blocks (256-body panels): from 21504
//     to 77824 bodies;
//  3  2 i-bodies per lane in one-wave blocks (128-body panels): up to
//     21504 bodies, where larger panels leave too few panel pairs to fill
//     the chip's 8192 wave slots;
//  4  variant 0 with the j-state rotated one lane per step by DPP instead of
//     carried in LDS (7 / K moves per pair): the ablation of the LDS
//     carriage (the same panel shape; the j-side sums are added in another
//     order, so it agrees with 0 to rounding).
// A one-wave task needs no barrier: the wave adds its own j-side sums.
// One-wave tasks are paced (pace): a launch of them is about one round of
// waves, and the SIMD's oldest-first issue would otherwise finish its waves
// one after another, leaving the last ones to run nearly alone; raising the
// priority of the waves that are behind makes them drain together (at 16384
// bodies 72.0 against 74.8 us for the whole pass, at 24576 bodies with 4
// i-bodies per lane 133.3 against 145.7 us).  With 4-wave blocks, whose
// launches are many rounds, it cost 1 to 3.5 % and is not used.
// Other shapes measured on MI355X and not kept: the rotated carriage with 2
// j-bodies per lane, 4 to 16 i-bodies per lane, 6 to 8 waves per SIMD, pair
// interleave widths 2 and 4 (the same as 1 under this register budget), 6 or
// all 8 i-masses in LDS, 2 i-bodies per lane in 2-wave blocks, 8 in 2-wave
// and one-wave blocks and 4 in 2-wave blocks (2 to 8 % slower than variant 1
// at 65536 to 262144 bodies, level at 393216), several
// one-wave tasks packed into one block (no gain), and loading the next
// sweep's j-bodies one sweep ahead (up to 5 % slower with 4 i-bodies per
// lane, no gain with 2).
#define NBODY_SYM_VARIANTS(X) \
  X(0, 8, 1, 4, 7, 1, 5, 8)   \
  X(1, 4, 1, 4, 8, 1, 0, 8)   \
  X(2, 4, 1, 1, 8, 1, 0, 8)   \
  X(3, 2, 1, 1, 8, 1, 0, 8)   \
  X(4, 8, 1, 4, 7, 1, 5, 0)

// Variants of the pass that also sums the potential (id, K, KP, waves,
// occupancy target, i-masses in LDS, JL as above); the ids are their own
// (nbody_accel_symmetric_potential), and variant v has the panel shape and
// j-state carriage of the plain variant v, so their xyz outputs are bitwise
// equal.  The potential sums cost registers: with 8 i-bodies per lane,
// 4 i-masses in LDS and 5 waves per SIMD (no spills); rotated instead, K = 8
// took ~96 VGPRs (266 ms at 2^20 bodies) or 80 with spills (216 ms), against
// 201 ms for variant 0.
#define NBODY_SYM_POT_VARIANTS(X) \
  X(0, 8, 1, 4, 5, 4, 8)          \
  X(1, 4, 1, 4, 8, 0, 8)          \
  X(2, 4, 1, 1, 8, 0, 8)          \
  X(3, 2, 1, 1, 8, 0, 8)

struct SymVariant {
  int K, KP, W;
};

const SymVariant kSym[] = {
#define X(id, K, KP, W, OCC, IL, ML, JL) {K, KP, W},
    NBODY_SYM_VARIANTS(X)
#undef X
};

const SymVariant kSymPot[] = {
#define X(id, K, KP, W, OCC, ML, JL) {K, KP, W},
    NBODY_SYM_POT_VARIANTS(X)
#undef X
};

const SymVariant &sym_table(int v, bool pot) { return pot ? kSymPot[v] : kSym[v]; }

}  // namespace

int symmetric_variant_count(bool pot) {
  return pot ? (int)(sizeof(kSymPot) / sizeof(kSymPot[0])) : (int)(sizeof(kSym) / sizeof(kSym[0]));
}

// Measured on MI355X (force-pass sweeps of every variant on Plummer spheres
// of 8192 to 524288 bodies, each call timed whole: panel pairs and reduce),
// all with the j-state in LDS: 2 i-bodies per lane in one-wave blocks up to
// ~21000 bodies (74.9 us at 16384 against 88.5 us for 4 i-bodies, and 85 to
// 96 us for the one-sided pass; 105.5 against 110.4 us at 20480, 122.1 against
// 112.5 us at 22528), 4 in one-wave blocks up to ~78000 (0.826 against 0.855
// ms for 4-wave blocks at 65536, 1.038 against 1.045 ms at 73728, 1.289
// against 1.228 ms at 81920), 4 in 4-wave blocks up to ~3e5 (3.04 against
// 3.30 ms at 131072; 12.07 against 12.29 ms at 262144, the same at 327680),
// 8 in 4-wave blocks above (26.7 against 27.0 ms at 393216, 46.9 against
// 47.8 ms at 2^19).  The potential variants follow the same split, with the
// same panel shapes and j-state carriage, so their xyz equal the plain
// pass's.
int symmetric_variant_for_n(int64_t n, bool pot) {
  (void)pot;
  return n <= 21504 ? 3 : n <= 77824 ? 2 : n <= 300000 ? 1 : 0;
}

int symmetric_panel(int v, bool pot) {
  const SymVariant &t = sym_table(v, pot);
  return kWave * t.W * t.K;
}

int64_t symmetric_panels(int64_t n, int v, bool pot) {
  const int64_t B = symmetric_panel(v, pot);
  return (n + B - 1) / B;
}

size_t symmetric_workspace_bytes(int64_t n, int v, bool pot) {
  if (n <= 0 || v < 0 || v >= symmetric_variant_count(pot)) return 0;
  const int64_t B = symmetric_panel(v, pot), P = symmetric_panels(n, v, pot);
  return (size_t)P * (size_t)P * (pot ? 4 : 3) * (size_t)B * sizeof(float);
}

bool symmetric_chunk_ok(int chunk_panels) {
  return chunk_panels > 0 && chunk_panels % kPanelTile == 0;
}

// Bytes of one chunk's slots: the largest over the chunks (the last full one).
static size_t chunk_slot_bytes(int64_t n, int v, bool pot, int chunk_panels) {
  const int64_t B = symmetric_panel(v, pot), P = symmetric_panels(n, v, pot);
  long long most = 0;
  for (int64_t c0 = 0; c0 < P; c0 += chunk_panels) {
    const SlotMap map{(int)c0, (int)std::min<int64_t>(P, c0 + chunk_panels)};
    most = std::max(most, map.slots());
  }
  // rounded up to 256 bytes, so that the second buffer starts aligned
  const size_t bytes = (size_t)most * (pot ? 4 : 3) * (size_t)B * sizeof(float);
  return (bytes + 255) & ~(size_t)255;
}

size_t symmetric_chunked_workspace_bytes(int64_t n, int v, bool pot, int chunk_panels) {
  if (n <= 0 || v < 0 || v >= symmetric_variant_count(pot) || !symmetric_chunk_ok(chunk_panels))
    return 0;
  const int64_t P = symmetric_panels(n, v, pot);
  // two buffers when there are two chunks or more (consecutive chunks run
  // at the same time on two queues)
  return chunk_slot_bytes(n, v, pot, chunk_panels) * (P > chunk_panels ? 2 : 1);
}

// The task kernel over the panel pairs with J in [c0, c1) (c0 a multiple of
// the tile side; [0, P) for the whole pass), writing the slots of that chunk.
static hipError_t launch_tasks_columns(const float *posmass, int n, float eps2, int v, bool pot,
                                       void *workspace, int c0, int c1, hipStream_t stream) {
  const int P = (int)symmetric_panels(n, v, pot);
  const long long first = first_pair_of_column(c0), last = first_pair_of_column(c1);
  const SlotMap map{c0, c1};
  float *part = reinterpret_cast<float *>(workspace);
  const float4 *pm = reinterpret_cast<const float4 *>(posmass);
  if (!pot) {
    switch (v) {
#define X(id, K, KP, W, OCC, IL, ML, JL)                                                      \
  case id:                                                                                     \
    return launch_pair_ranges(P, first, last, W * kWave, [&](const PanelOrder &o, long long b) { \
      hipLaunchKernelGGL((symmetric_task_kernel<K, KP, W, OCC, IL, false, ML, JL>),            \
                         dim3((unsigned)b), dim3(W * kWave), 0, stream, pm, n, o, map, eps2,   \
                         part);                                                                \
    });
      NBODY_SYM_VARIANTS(X)
#undef X
      default:
        return hipErrorInvalidValue;
    }
  }
  switch (v) {
#define X(id, K, KP, W, OCC, ML, JL)                                                          \
  case id:                                                                                     \
    return launch_pair_ranges(P, first, last, W * kWave, [&](const PanelOrder &o, long long b) { \
      hipLaunchKernelGGL((symmetric_task_kernel<K, KP, W, OCC, 1, true, ML, JL>),              \
                         dim3((unsigned)b), dim3(W * kWave), 0, stream, pm, n, o, map, eps2,   \
                         part);                                                                \
    });
    NBODY_SYM_POT_VARIANTS(X)
#undef X
    default:
      return hipErrorInvalidValue;
  }
}

// The reduce of the chunk [c0, c1): the bodies of panels below c1.
static hipError_t launch_reduce_columns(int n, float G, float *accel, int v, bool pot,
                                        const void *workspace, int c0, int c1,
                                        hipStream_t stream) {
  const int B = symmetric_panel(v, pot);
  const int P = (int)symmetric_panels(n, v, pot);
  const int touched = (int)std::min<int64_t>(n, (int64_t)c1 * B);
  const SlotMap map{c0, c1};
  const int last = c1 == P;
  const float *part = reinterpret_cast<const float *>(workspace);
  float4 *out = reinterpret_cast<float4 *>(accel);
  const int nc = pot ? 4 : 3;
  // one thread per (body, component) once that alone makes 16384 waves (two
  // rounds of the chip), the split form below that; measured on MI355X, the
  // walk took 1.135 against 1.172 ms at 2^20 bodies and 0.295 against 0.309
  // ms at 2^19, and the split form 4.4 against 7.6 us at 16384 bodies
  // (where one thread per body and component gives only 768 waves)
  if ((int64_t)touched * nc >= (int64_t)16384 * kWave) {
    const dim3 grid((touched + 255) / 256, nc);
    if (pot)
      hipLaunchKernelGGL(symmetric_reduce_walk_kernel<true>, grid, dim3(256), 0, stream, part,
                         touched, B, map, last, G, out);
    else
      hipLaunchKernelGGL(symmetric_reduce_walk_kernel<false>, grid, dim3(256), 0, stream, part,
                         touched, B, map, last, G, out);
    return hipGetLastError();
  }
  const dim3 grid((touched + kWave - 1) / kWave, nc);
  if (pot)
    hipLaunchKernelGGL(symmetric_reduce_kernel<true>, grid, dim3(kReduceWaves * kWave), 0,
                       stream, part, touched, B, map, last, G, out);
  else
    hipLaunchKernelGGL(symmetric_reduce_kernel<false>, grid, dim3(kReduceWaves * kWave), 0,
                       stream, part, touched, B, map, last, G, out);
  return hipGetLastError();
}

hipError_t launch_symmetric_tasks(const float *posmass, int n, float eps2, int v, bool pot,
                                  void *workspace, hipStream_t stream) {
  return launch_tasks_columns(posmass, n, eps2, v, pot, workspace, 0,
                              (int)symmetric_panels(n, v, pot), stream);
}

hipError_t launch_symmetric_reduce(int n, float G, float *accel, int v, bool pot,
                                   const void *workspace, hipStream_t stream) {
  return launch_reduce_columns(n, G, accel, v, pot, workspace, 0,
                               (int)symmetric_panels(n, v, pot), stream);
}

hipError_t launch_symmetric(const float *posmass, int n, float G, float eps2, float *accel,
                            int v, bool pot, void *workspace, hipStream_t stream) {
  const hipError_t e = launch_symmetric_tasks(posmass, n, eps2, v, pot, workspace, stream);
  if (e != hipSuccess) return e;
  return launch_symmetric_reduce(n, G, accel, v, pot, workspace, stream);
}

// The library's second queue on each GPU for the chunked pass: a side stream
// (default priority) and a pool of events, made on first use with that GPU
// current and kept until the process ends.  The mutex also keeps the
// enqueue sequence of one chunked call from interleaving with another's.
namespace {

constexpr int kMaxSideDevices = 64;

struct SideQueue {
  hipStream_t stream = nullptr;
  std::vector<hipEvent_t> events;
};

std::mutex g_side_mutex;
SideQueue g_side[kMaxSideDevices];

// Under g_side_mutex: the current GPU's side queue with at least `events`
// events.
hipError_t side_queue(int events, SideQueue *&q) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxSideDevices) return hipErrorInvalidDevice;
  q = &g_side[dev];
  if (!q->stream) {
    e = hipStreamCreateWithFlags(&q->stream, hipStreamNonBlocking);
    if (e != hipSuccess) {
      q->stream = nullptr;
      return e;
    }
  }
  while ((int)q->events.size() < events) {
    hipEvent_t ev = nullptr;
    e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
    if (e != hipSuccess) return e;
    q->events.push_back(ev);
  }
  return hipSuccess;
}

}  // namespace

// Chunk c = [c0, c0 + C) runs on the caller's stream for even c and on the
// side queue for odd c, in slot buffer c % 2: its panel-pair kernel may run
// alongside the previous chunk's, so the tail of one launch is filled by the
// next instead of leaving CUs idle.  Its reduce waits for the previous
// chunk's reduce (event c - 1), since both add into the same running sums;
// the next chunk on the same queue, which reuses the buffer, follows the
// reduce in stream order.  The caller's stream waits for the last event, and
// every side-queue operation is ordered before it.
hipError_t launch_symmetric_chunked(const float *posmass, int n, float G, float eps2,
                                    float *accel, int v, bool pot, int chunk_panels,
                                    void *workspace, hipStream_t stream) {
  const int P = (int)symmetric_panels(n, v, pot);
  const int chunks = (P + chunk_panels - 1) / chunk_panels;
  if (chunks == 1) {
    const hipError_t e = launch_tasks_columns(posmass, n, eps2, v, pot, workspace, 0, P, stream);
    if (e != hipSuccess) return e;
    return launch_reduce_columns(n, G, accel, v, pot, workspace, 0, P, stream);
  }
  const size_t half = chunk_slot_bytes(n, v, pot, chunk_panels);
  std::lock_guard<std::mutex> lock(g_side_mutex);
  SideQueue *q = nullptr;
  hipError_t e = side_queue(chunks + 1, q);
  if (e != hipSuccess) return e;
  hipEvent_t fork = q->events[chunks];
  e = hipEventRecord(fork, stream);
  if (e == hipSuccess) e = hipStreamWaitEvent(q->stream, fork, 0);
  for (int c = 0; c < chunks && e == hipSuccess; ++c) {
    const int c0 = c * chunk_panels, c1 = std::min(P, c0 + chunk_panels);
    const hipStream_t s = (c % 2 == 0) ? stream : q->stream;
    void *buf = static_cast<char *>(workspace) + (c % 2) * half;
    e = launch_tasks_columns(posmass, n, eps2, v, pot, buf, c0, c1, s);
    if (e == hipSuccess && c > 0) e = hipStreamWaitEvent(s, q->events[c - 1], 0);
    if (e == hipSuccess) e = launch_reduce_columns(n, G, accel, v, pot, buf, c0, c1, s);
    if (e == hipSuccess) e = hipEventRecord(q->events[c], s);
  }
  if (e == hipSuccess) e = hipStreamWaitEvent(stream, q->events[chunks - 1], 0);
  return e;
}

}  // namespace nbody
