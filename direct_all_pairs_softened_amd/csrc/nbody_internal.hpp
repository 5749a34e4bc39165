// Host-side launchers of libnbody, shared between the kernel translation
// units and the C ABI layer.  Internal header: not part of the C ABI.
//
// Every launcher assumes its arguments were validated by the C ABI layer
// (n >= 1, pointers non-null, aligned and disjoint as documented in nbody.h)
// and returns the hipError_t of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nbody {

// HIP counts a launch's size in work-items with 32 bits per grid dimension,
// so one launch holds at most (2^32 - 1) / threads blocks.  Launchers whose
// grid can grow past that (one block per panel pair, or 16 to 32 threads
// per body) split it into several launches of at most launch_block_cap
// blocks each; every block computes the same thing in any launch, so the
// split changes no result.  set_launch_block_cap lowers the cap (0 restores
// the hardware limit): a testing aid that makes small inputs split.
long long launch_block_cap(int threads_per_block);
void set_launch_block_cap(long long blocks);

// Force-pass tiling of one compiled variant.
struct ForceVariant {
  int bodies_per_lane;  // K: i-bodies held in registers by each lane
  int tile;             // T: j-bodies per LDS tile (two-level summation chunk)
  int waves;            // waves per block
  int split;            // S: j-parts per block (waves / S waves per part)
  int unroll;           // unroll of the inner j loop
  int staging;          // 0: LDS tiles; 1: scalar loads of j; 2: vector loads of j
  int lane_groups;      // LG: lane groups per wave, each taking every LG-th j of a tile
};

int force_variant_count();
const ForceVariant *force_variant(int v);
int force_variant_for_n(int64_t n);

enum class Layout { Aos4, Aos3, Soa };

struct BodyArrays {
  // Aos4
  const float *posmass = nullptr;
  float *accel4 = nullptr;
  // Aos3
  const float *pos3 = nullptr;
  const float *mass = nullptr;
  float *accel3 = nullptr;
  // Soa
  const float *x = nullptr, *y = nullptr, *z = nullptr, *m = nullptr;
  float *ax = nullptr, *ay = nullptr, *az = nullptr;
};

// i side: bodies [i0, i0 + ni); output row r belongs to body i0 + r.
hipError_t launch_force(int variant, Layout layout, const BodyArrays &b, int n, int i0, int ni,
                        float G, float eps2, hipStream_t stream);

// One-sided pass that also stores Phi_i = -G sum_{j != i} m_j / sqrt(r^2 + eps^2)
// in accel.w (variant chosen by n).
hipError_t launch_force_potential(const float *posmass, int n, float G, float eps2,
                                  float *accel, hipStream_t stream);

// Two-pass decomposition over j chunks.
size_t splitj_workspace_bytes(int64_t n, int64_t j_chunk);
hipError_t launch_splitj(const float *posmass, int n, float G, float eps2, float *accel,
                         int j_chunk, void *workspace, hipStream_t stream);
bool splitj_tree_shape_ok(int64_t j_chunk, int terms);
size_t splitj_tree_workspace_bytes(int64_t n, int64_t j_chunk, int terms);
hipError_t launch_splitj_tree(const float *posmass, int n, float G, float eps2, float *accel,
                              int j_chunk, int terms, void *workspace, hipStream_t stream);

// Pair-symmetric force pass (each pair once, applied to both bodies).  pot
// selects the variants that also store Phi_i = -G sum_{j != i} m_j /
// sqrt(r^2 + eps^2) in accel.w; their variant ids are a table of their own.
int symmetric_variant_count(bool pot);
int symmetric_variant_for_n(int64_t n, bool pot);
int symmetric_panel(int v, bool pot);
int64_t symmetric_panels(int64_t n, int v, bool pot);
size_t symmetric_workspace_bytes(int64_t n, int v, bool pot);
hipError_t launch_symmetric(const float *posmass, int n, float G, float eps2, float *accel,
                            int v, bool pot, void *workspace, hipStream_t stream);
// The two kernels of launch_symmetric: the panel-pair tasks (posmass ->
// workspace) and the reduce (workspace -> accel).
hipError_t launch_symmetric_tasks(const float *posmass, int n, float eps2, int v, bool pot,
                                  void *workspace, hipStream_t stream);
hipError_t launch_symmetric_reduce(int n, float G, float *accel, int v, bool pot,
                                   const void *workspace, hipStream_t stream);
// The same pass in column chunks of chunk_panels panels (a positive multiple
// of the panel-pair tile side, 32): per chunk a task launch and a reduce
// launch; bitwise equal to launch_symmetric, with a workspace of one
// chunk's slots.
bool symmetric_chunk_ok(int chunk_panels);
size_t symmetric_chunked_workspace_bytes(int64_t n, int v, bool pot, int chunk_panels);
hipError_t launch_symmetric_chunked(const float *posmass, int n, float G, float eps2,
                                    float *accel, int v, bool pot, int chunk_panels,
                                    void *workspace, hipStream_t stream);

// Integrator.
// closing half-kick of a step and kick-drift of the next, fused (h = dt / 2)
hipError_t launch_kick_leapfrog(float *posmass, float *vel, const float *accel, float dt, int n,
                                hipStream_t stream);
hipError_t launch_leapfrog(float *posmass, float *vel, const float *accel, float dt, int n,
                           hipStream_t stream);
hipError_t launch_kick(float *vel, const float *accel, float h, int n, hipStream_t stream);

// Energy.
size_t energy_workspace_bytes(int64_t n);
int64_t energy_pair_tasks(int64_t n);  // blocks of the pair pass
size_t energy_from_potential_workspace_bytes(int64_t n);
hipError_t launch_energy_from_potential(const float *posmass, const float *vel,
                                        const float *accel, int n, void *workspace,
                                        double *stats, hipStream_t stream);
hipError_t launch_energy(const float *posmass, const float *vel, int n, float G, float eps2,
                         void *workspace, double *stats, hipStream_t stream);
// The allocation-free energy entry point's static device scratch: its size,
// and its device address on the current GPU (looked up once per GPU).
constexpr size_t kEnergyStaticScratchBytes = (size_t)16 << 20;
hipError_t energy_static_scratch(void **ptr);

}  // namespace nbody
