// C ABI of libnbody.so (declared in include/nbody.h): argument validation and
// dispatch to the kernel launchers.  Every check runs before anything is
// enqueued, and none of them touches device memory or the HIP runtime, so
// invalid calls fail the same way with or without a GPU.
#include "nbody.h"

#include <math.h>
#include <stdint.h>

#include <atomic>
#include <vector>

#include "nbody_internal.hpp"

static_assert(NBODY_ENERGY_STATIC_SCRATCH_BYTES == nbody::kEnergyStaticScratchBytes,
              "the header's scratch size must match the library's");

namespace nbody {

namespace {
std::atomic<long long> g_launch_block_cap{0};
}  // namespace

long long launch_block_cap(int threads_per_block) {
  const long long hw = 0xFFFFFFFFLL / threads_per_block;
  const long long test = g_launch_block_cap.load(std::memory_order_relaxed);
  return test > 0 && test < hw ? test : hw;
}

void set_launch_block_cap(long long blocks) {
  g_launch_block_cap.store(blocks > 0 ? blocks : 0, std::memory_order_relaxed);
}

}  // namespace nbody

namespace {

using nbody::BodyArrays;
using nbody::Layout;

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// [a, a + na) and [b, b + nb) share at least one byte.
bool overlap(const void *a, size_t na, const void *b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return na && nb && x < y + nb && y < x + na;
}

bool n_ok(int64_t n) { return n >= 0 && n <= NBODY_MAX_N; }

int check_consts(float G, float eps2) {
  if (!isfinite(G) || !isfinite(eps2) || !(eps2 > 0.0f)) return NBODY_ERR_INVALID_ARG;
  return NBODY_OK;
}

// A failed runtime call is reported through the status alone: its error is
// also consumed from the thread's last-error state, so that the caller's own
// next error check does not see it again (a fault that leaves the device
// unusable stays reported by every later call anyway).
int hip_status(hipError_t e) {
  if (e == hipSuccess) return NBODY_OK;
  (void)hipGetLastError();
  return NBODY_ERR_HIP;
}

hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

// The checks of the one-sided float4 pass; NBODY_OK with n == 0 means there
// is nothing to launch.
int force_aos4_check(const float *posmass, int64_t n, float G, float eps2,
                     const float *accel_out, int variant) {
  if (!n_ok(n)) return NBODY_ERR_INVALID_ARG;
  if (int s = check_consts(G, eps2)) return s;
  if (!nbody::force_variant(variant)) return NBODY_ERR_INVALID_ARG;
  if (n == 0) return NBODY_OK;
  if (!posmass || !accel_out) return NBODY_ERR_INVALID_ARG;
  if (!aligned(posmass, 16) || !aligned(accel_out, 16)) return NBODY_ERR_ALIGNMENT;
  const size_t bytes = (size_t)n * 16;
  if (overlap(posmass, bytes, accel_out, bytes)) return NBODY_ERR_ALIAS;
  return NBODY_OK;
}

int force_aos4(const float *posmass, int64_t n, float G, float eps2, float *accel_out,
               int variant, void *stream) {
  if (int s = force_aos4_check(posmass, n, G, eps2, accel_out, variant)) return s;
  if (n == 0) return NBODY_OK;
  BodyArrays b;
  b.posmass = posmass;
  b.accel4 = accel_out;
  return hip_status(nbody::launch_force(variant, Layout::Aos4, b, (int)n, 0, (int)n, G, eps2,
                                        as_stream(stream)));
}

}  // namespace

extern "C" {

const char *nbody_status_string(int status) {
  switch (status) {
    case NBODY_OK:
      return "ok";
    case NBODY_ERR_INVALID_ARG:
      return "invalid argument (null pointer, body count out of range, eps2 <= 0 or a "
             "non-finite constant, unknown variant or bad split size)";
    case NBODY_ERR_ALIGNMENT:
      return "misaligned array (float4 arrays need 16 bytes, float arrays 4)";
    case NBODY_ERR_ALIAS:
      return "an output array overlaps an array it must not";
    case NBODY_ERR_WORKSPACE:
      return "workspace missing or too small";
    case NBODY_ERR_HIP:
      return "HIP launch or runtime error";
    default:
      return "unknown status";
  }
}

int nbody_abi_version(void) { return NBODY_ABI_VERSION; }

int nbody_accel_variant_count(void) { return nbody::force_variant_count(); }

int nbody_accel_variant_info(int v, int *bodies_per_lane, int *tile, int *waves_per_block,
                             int *split, int *staging, int *unroll, int *lane_groups) {
  const nbody::ForceVariant *fv = nbody::force_variant(v);
  if (!fv) return NBODY_ERR_INVALID_ARG;
  if (bodies_per_lane) *bodies_per_lane = fv->bodies_per_lane;
  if (tile) *tile = fv->tile;
  if (waves_per_block) *waves_per_block = fv->waves;
  if (split) *split = fv->split;
  if (staging) *staging = fv->staging;
  if (unroll) *unroll = fv->unroll;
  if (lane_groups) *lane_groups = fv->lane_groups;
  return NBODY_OK;
}

int nbody_accel_variant_for_n(int64_t n) { return nbody::force_variant_for_n(n); }

int nbody_accel(const float *posmass, int64_t n, float G, float eps2, float *accel_out,
                void *stream) {
  return force_aos4(posmass, n, G, eps2, accel_out, nbody::force_variant_for_n(n), stream);
}

int nbody_accel_variant(const float *posmass, int64_t n, float G, float eps2, float *accel_out,
                        int variant, void *stream) {
  return force_aos4(posmass, n, G, eps2, accel_out, variant, stream);
}

int nbody_accel_potential(const float *posmass, int64_t n, float G, float eps2,
                          float *accel_out, void *stream) {
  if (!n_ok(n)) return NBODY_ERR_INVALID_ARG;
  if (int s = check_consts(G, eps2)) return s;
  if (n == 0) return NBODY_OK;
  if (!posmass || !accel_out) return NBODY_ERR_INVALID_ARG;
  if (!aligned(posmass, 16) || !aligned(accel_out, 16)) return NBODY_ERR_ALIGNMENT;
  const size_t bytes = (size_t)n * 16;
  if (overlap(posmass, bytes, accel_out, bytes)) return NBODY_ERR_ALIAS;
  return hip_status(
      nbody::launch_force_potential(posmass, (int)n, G, eps2, accel_out, as_stream(stream)));
}

int nbody_accel_range(const float *posmass, int64_t n, int64_t i0, int64_t ni, float G,
                      float eps2, float *accel_out, int variant, void *stream) {
  if (!n_ok(n) || i0 < 0 || ni < 0 || i0 > n || ni > n - i0) return NBODY_ERR_INVALID_ARG;
  if (int s = check_consts(G, eps2)) return s;
  const int v = variant < 0 ? nbody::force_variant_for_n(ni) : variant;
  if (!nbody::force_variant(v)) return NBODY_ERR_INVALID_ARG;
  if (ni == 0) return NBODY_OK;
  if (!posmass || !accel_out) return NBODY_ERR_INVALID_ARG;
  if (!aligned(posmass, 16) || !aligned(accel_out, 16)) return NBODY_ERR_ALIGNMENT;
  if (overlap(posmass, (size_t)n * 16, accel_out, (size_t)ni * 16)) return NBODY_ERR_ALIAS;
  BodyArrays b;
  b.posmass = posmass;
  b.accel4 = accel_out;
  return hip_status(nbody::launch_force(v, Layout::Aos4, b, (int)n, (int)i0, (int)ni, G, eps2,
                                        as_stream(stream)));
}

int nbody_accel_f3aos(const float *pos, const float *mass, int64_t n, float G, float eps2,
                      float *accel_out, void *stream) {
  if (!n_ok(n)) return NBODY_ERR_INVALID_ARG;
  if (int s = check_consts(G, eps2)) return s;
  if (n == 0) return NBODY_OK;
  if (!pos || !mass || !accel_out) return NBODY_ERR_INVALID_ARG;
  if (!aligned(pos, 4) || !aligned(mass, 4) || !aligned(accel_out, 4)) return NBODY_ERR_ALIGNMENT;
  const size_t b3 = (size_t)n * 12, b1 = (size_t)n * 4;
  if (overlap(accel_out, b3, pos, b3) || overlap(accel_out, b3, mass, b1)) return NBODY_ERR_ALIAS;
  BodyArrays b;
  b.pos3 = pos;
  b.mass = mass;
  b.accel3 = accel_out;
  return hip_status(nbody::launch_force(nbody::force_variant_for_n(n), Layout::Aos3, b, (int)n,
                                        0, (int)n, G, eps2, as_stream(stream)));
}

int nbody_accel_soa(const float *x, const float *y, const float *z, const float *m, int64_t n,
                    float G, float eps2, float *ax, float *ay, float *az, void *stream) {
  if (!n_ok(n)) return NBODY_ERR_INVALID_ARG;
  if (int s = check_consts(G, eps2)) return s;
  if (n == 0) return NBODY_OK;
  const float *in[4] = {x, y, z, m};
  float *out[3] = {ax, ay, az};
  for (const float *p : in)
    if (!p) return NBODY_ERR_INVALID_ARG;
  for (const float *p : out)
    if (!p) return NBODY_ERR_INVALID_ARG;
  for (const float *p : in)
    if (!aligned(p, 4)) return NBODY_ERR_ALIGNMENT;
  for (const float *p : out)
    if (!aligned(p, 4)) return NBODY_ERR_ALIGNMENT;
  const size_t b1 = (size_t)n * 4;
  for (int o = 0; o < 3; ++o) {
    for (const float *p : in)
      if (overlap(out[o], b1, p, b1)) return NBODY_ERR_ALIAS;
    for (int o2 = o + 1; o2 < 3; ++o2)
      if (overlap(out[o], b1, out[o2], b1)) return NBODY_ERR_ALIAS;
  }
  BodyArrays b;
  b.x = x;
  b.y = y;
  b.z = z;
  b.m = m;
  b.ax = ax;
  b.ay = ay;
  b.az = az;
  return hip_status(nbody::launch_force(nbody::force_variant_for_n(n), Layout::Soa, b, (int)n, 0,
                                        (int)n, G, eps2, as_stream(stream)));
}

size_t nbody_accel_splitj_workspace_bytes(int64_t n, int64_t j_chunk) {
  if (!n_ok(n)) return 0;
  return nbody::splitj_workspace_bytes(n, j_chunk);
}

int nbody_accel_splitj(const float *posmass, int64_t n, float G, float eps2, float *accel_out,
                       int64_t j_chunk, void *workspace, size_t workspace_bytes, void *stream) {
  if (!n_ok(n)) return NBODY_ERR_INVALID_ARG;
  if (int s = check_consts(G, eps2)) return s;
  if (j_chunk < 32 || j_chunk % 32 != 0 || j_chunk > NBODY_MAX_N) return NBODY_ERR_INVALID_ARG;
  if (n == 0) return NBODY_OK;
  // the chunk index is the grid's y dimension
  if ((n + j_chunk - 1) / j_chunk > 65535) return NBODY_ERR_INVALID_ARG;
  if (!posmass || !accel_out) return NBODY_ERR_INVALID_ARG;
  if (!aligned(posmass, 16) || !aligned(accel_out, 16)) return NBODY_ERR_ALIGNMENT;
  const size_t need = nbody::splitj_workspace_bytes(n, j_chunk);
  if (!workspace || workspace_bytes < need) return NBODY_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return NBODY_ERR_ALIGNMENT;
  const size_t bytes = (size_t)n * 16;
  if (overlap(posmass, bytes, accel_out, bytes) || overlap(workspace, need, posmass, bytes) ||
      overlap(workspace, need, accel_out, bytes))
    return NBODY_ERR_ALIAS;
  return hip_status(nbody::launch_splitj(posmass, (int)n, G, eps2, accel_out, (int)j_chunk,
                                         workspace, as_stream(stream)));
}

size_t nbody_accel_splitj_tree_workspace_bytes(int64_t n, int64_t j_chunk, int terms) {
  if (!n_ok(n)) return 0;
  return nbody::splitj_tree_workspace_bytes(n, j_chunk, terms);
}

int nbody_accel_splitj_tree(const float *posmass, int64_t n, float G, float eps2,
                            float *accel_out, int64_t j_chunk, int terms, void *workspace,
                            size_t workspace_bytes, void *stream) {
  if (!n_ok(n)) return NBODY_ERR_INVALID_ARG;
  if (int s = check_consts(G, eps2)) return s;
  if (!nbody::splitj_tree_shape_ok(j_chunk, terms)) return NBODY_ERR_INVALID_ARG;
  if (n == 0) return NBODY_OK;
  // the chunk index is the grid's y dimension
  if ((n + j_chunk - 1) / j_chunk > 65535) return NBODY_ERR_INVALID_ARG;
  if (!posmass || !accel_out) return NBODY_ERR_INVALID_ARG;
  if (!aligned(posmass, 16) || !aligned(accel_out, 16)) return NBODY_ERR_ALIGNMENT;
  const size_t need = nbody::splitj_tree_workspace_bytes(n, j_chunk, terms);
  if (!workspace || workspace_bytes < need) return NBODY_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return NBODY_ERR_ALIGNMENT;
  const size_t bytes = (size_t)n * 16;
  if (overlap(posmass, bytes, accel_out, bytes) || overlap(workspace, need, posmass, bytes) ||
      overlap(workspace, need, accel_out, bytes))
    return NBODY_ERR_ALIAS;
  return hip_status(nbody::launch_splitj_tree(posmass, (int)n, G, eps2, accel_out, (int)j_chunk,
                                              terms, workspace, as_stream(stream)));
}

static int sym_variant(int v, int64_t n, bool pot) {
  return v < 0 ? nbody::symmetric_variant_for_n(n, pot) : v;
}

static size_t sym_workspace_bytes(int64_t n, int variant, bool pot) {
  const int v = sym_variant(variant, n, pot);
  if (!n_ok(n) || v >= nbody::symmetric_variant_count(pot)) return 0;
  return nbody::symmetric_workspace_bytes(n, v, pot);
}

// Checks shared by the pair-symmetric entry points.  A phase that does not
// read posmass, or does not write accel_out, passes it as null with want_pm
// or want_out false.  NBODY_OK with n == 0 means there is nothing to launch.
static int sym_check(const float *posmass, int64_t n, float G, float eps2,
                     const float *accel_out, int v, bool pot, const void *workspace,
                     size_t workspace_bytes, bool want_pm, bool want_out,
                     int chunk_panels = 0) {
  if (!n_ok(n)) return NBODY_ERR_INVALID_ARG;
  if (int s = check_consts(G, eps2)) return s;
  if (v >= nbody::symmetric_variant_count(pot)) return NBODY_ERR_INVALID_ARG;
  if (n == 0) return NBODY_OK;
  const int64_t P = nbody::symmetric_panels(n, v, pot);
  // one block per panel pair, the grid rounded up to whole XCD stretches
  if (P * (P + 1) / 2 > INT32_MAX - 8) return NBODY_ERR_INVALID_ARG;
  if ((want_pm && !posmass) || (want_out && !accel_out)) return NBODY_ERR_INVALID_ARG;
  if ((want_pm && !aligned(posmass, 16)) || (want_out && !aligned(accel_out, 16)))
    return NBODY_ERR_ALIGNMENT;
  const size_t need = chunk_panels > 0
                          ? nbody::symmetric_chunked_workspace_bytes(n, v, pot, chunk_panels)
                          : nbody::symmetric_workspace_bytes(n, v, pot);
  if (!workspace || workspace_bytes < need) return NBODY_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return NBODY_ERR_ALIGNMENT;
  const size_t bytes = (size_t)n * 16;
  if ((want_pm && want_out && overlap(posmass, bytes, accel_out, bytes)) ||
      (want_pm && overlap(workspace, need, posmass, bytes)) ||
      (want_out && overlap(workspace, need, accel_out, bytes)))
    return NBODY_ERR_ALIAS;
  return NBODY_OK;
}

static int sym_pass(const float *posmass, int64_t n, float G, float eps2, float *accel_out,
                    int variant, bool pot, void *workspace, size_t workspace_bytes,
                    void *stream) {
  const int v = sym_variant(variant, n, pot);
  if (int s = sym_check(posmass, n, G, eps2, accel_out, v, pot, workspace, workspace_bytes, true,
                        true))
    return s;
  if (n == 0) return NBODY_OK;
  return hip_status(nbody::launch_symmetric(posmass, (int)n, G, eps2, accel_out, v, pot,
                                            workspace, as_stream(stream)));
}

int nbody_accel_symmetric_variant_count(void) { return nbody::symmetric_variant_count(false); }

int nbody_accel_symmetric_variant_for_n(int64_t n) {
  return nbody::symmetric_variant_for_n(n, false);
}

int nbody_accel_symmetric_panel(int variant) {
  if (variant < 0 || variant >= nbody::symmetric_variant_count(false))
    return NBODY_ERR_INVALID_ARG;
  return nbody::symmetric_panel(variant, false);
}

size_t nbody_accel_symmetric_workspace_bytes(int64_t n, int variant) {
  return sym_workspace_bytes(n, variant, false);
}

int nbody_accel_symmetric(const float *posmass, int64_t n, float G, float eps2,
                          float *accel_out, int variant, void *workspace,
                          size_t workspace_bytes, void *stream) {
  return sym_pass(posmass, n, G, eps2, accel_out, variant, false, workspace, workspace_bytes,
                  stream);
}

static int chunk_of(int chunk_panels) {
  return chunk_panels == 0 ? NBODY_SYMMETRIC_DEFAULT_CHUNK : chunk_panels;
}

size_t nbody_accel_symmetric_chunked_workspace_bytes(int64_t n, int variant, int chunk_panels) {
  const int v = sym_variant(variant, n, false);
  if (!n_ok(n) || v >= nbody::symmetric_variant_count(false) ||
      !nbody::symmetric_chunk_ok(chunk_of(chunk_panels)))
    return 0;
  return nbody::symmetric_chunked_workspace_bytes(n, v, false, chunk_of(chunk_panels));
}

int nbody_accel_symmetric_chunked(const float *posmass, int64_t n, float G, float eps2,
                                  float *accel_out, int variant, int chunk_panels,
                                  void *workspace, size_t workspace_bytes, void *stream) {
  const int v = sym_variant(variant, n, false);
  const int c = chunk_of(chunk_panels);
  if (!nbody::symmetric_chunk_ok(c)) return NBODY_ERR_INVALID_ARG;
  if (int s = sym_check(posmass, n, G, eps2, accel_out, v, false, workspace, workspace_bytes,
                        true, true, c))
    return s;
  if (n == 0) return NBODY_OK;
  return hip_status(nbody::launch_symmetric_chunked(posmass, (int)n, G, eps2, accel_out, v,
                                                    false, c, workspace, as_stream(stream)));
}

int nbody_accel_symmetric_tasks(const float *posmass, int64_t n, float eps2, int variant,
                                void *workspace, size_t workspace_bytes, void *stream) {
  const int v = sym_variant(variant, n, false);
  if (int s = sym_check(posmass, n, 1.0f, eps2, nullptr, v, false, workspace, workspace_bytes,
                        true, false))
    return s;
  if (n == 0) return NBODY_OK;
  return hip_status(nbody::launch_symmetric_tasks(posmass, (int)n, eps2, v, false, workspace,
                                                  as_stream(stream)));
}

int nbody_accel_symmetric_reduce(int64_t n, float G, float *accel_out, int variant,
                                 const void *workspace, size_t workspace_bytes, void *stream) {
  const int v = sym_variant(variant, n, false);
  if (int s = sym_check(nullptr, n, G, 1.0f, accel_out, v, false, workspace, workspace_bytes,
                        false, true))
    return s;
  if (n == 0) return NBODY_OK;
  return hip_status(nbody::launch_symmetric_reduce((int)n, G, accel_out, v, false, workspace,
                                                   as_stream(stream)));
}

int nbody_accel_symmetric_potential_variant_count(void) {
  return nbody::symmetric_variant_count(true);
}

int nbody_accel_symmetric_potential_variant_for_n(int64_t n) {
  return nbody::symmetric_variant_for_n(n, true);
}

int nbody_accel_symmetric_potential_panel(int variant) {
  if (variant < 0 || variant >= nbody::symmetric_variant_count(true))
    return NBODY_ERR_INVALID_ARG;
  return nbody::symmetric_panel(variant, true);
}

size_t nbody_accel_symmetric_potential_workspace_bytes(int64_t n, int variant) {
  return sym_workspace_bytes(n, variant, true);
}

int nbody_accel_symmetric_potential(const float *posmass, int64_t n, float G, float eps2,
                                    float *accel_out, int variant, void *workspace,
                                    size_t workspace_bytes, void *stream) {
  return sym_pass(posmass, n, G, eps2, accel_out, variant, true, workspace, workspace_bytes,
                  stream);
}

int nbody_leapfrog_step(float *posmass, float *vel, const float *accel, float dt, int64_t n,
                        void *stream) {
  if (!n_ok(n) || !isfinite(dt)) return NBODY_ERR_INVALID_ARG;
  if (n == 0) return NBODY_OK;
  if (!posmass || !vel || !accel) return NBODY_ERR_INVALID_ARG;
  if (!aligned(posmass, 16) || !aligned(vel, 16) || !aligned(accel, 16))
    return NBODY_ERR_ALIGNMENT;
  const size_t bytes = (size_t)n * 16;
  if (overlap(posmass, bytes, vel, bytes) || overlap(posmass, bytes, accel, bytes) ||
      overlap(vel, bytes, accel, bytes))
    return NBODY_ERR_ALIAS;
  return hip_status(nbody::launch_leapfrog(posmass, vel, accel, dt, (int)n, as_stream(stream)));
}

int nbody_kick(float *vel, const float *accel, float h, int64_t n, void *stream) {
  if (!n_ok(n) || !isfinite(h)) return NBODY_ERR_INVALID_ARG;
  if (n == 0) return NBODY_OK;
  if (!vel || !accel) return NBODY_ERR_INVALID_ARG;
  if (!aligned(vel, 16) || !aligned(accel, 16)) return NBODY_ERR_ALIGNMENT;
  const size_t bytes = (size_t)n * 16;
  if (overlap(vel, bytes, accel, bytes)) return NBODY_ERR_ALIAS;
  return hip_status(nbody::launch_kick(vel, accel, h, (int)n, as_stream(stream)));
}

size_t nbody_energy_from_potential_workspace_bytes(int64_t n) {
  if (!n_ok(n)) return 0;
  return nbody::energy_from_potential_workspace_bytes(n);
}

int nbody_energy_from_potential(const float *posmass, const float *vel, const float *accel_pot,
                                int64_t n, void *workspace, size_t workspace_bytes,
                                double *stats_out, void *stream) {
  if (!n_ok(n)) return NBODY_ERR_INVALID_ARG;
  if (n == 0) return NBODY_OK;
  if (!posmass || !vel || !accel_pot || !stats_out) return NBODY_ERR_INVALID_ARG;
  if (!aligned(posmass, 16) || !aligned(vel, 16) || !aligned(accel_pot, 16) ||
      !aligned(stats_out, 8))
    return NBODY_ERR_ALIGNMENT;
  const size_t need = nbody::energy_from_potential_workspace_bytes(n);
  if (!workspace || workspace_bytes < need) return NBODY_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return NBODY_ERR_ALIGNMENT;
  const size_t bytes = (size_t)n * 16, sb = 8 * sizeof(double);
  const void *in[3] = {posmass, vel, accel_pot};
  for (const void *p : in)
    if (overlap(workspace, need, p, bytes) || overlap(stats_out, sb, p, bytes))
      return NBODY_ERR_ALIAS;
  if (overlap(workspace, need, stats_out, sb)) return NBODY_ERR_ALIAS;
  return hip_status(nbody::launch_energy_from_potential(posmass, vel, accel_pot, (int)n, workspace,
                                                        stats_out, as_stream(stream)));
}

int nbody_energy_static(const float *posmass, const float *vel, int64_t n, float G, float eps2,
                        double *stats_out, void *stream) {
  if (!n_ok(n)) return NBODY_ERR_INVALID_ARG;
  if (int s = check_consts(G, eps2)) return s;
  if (n == 0) return NBODY_OK;  // stats_out is left untouched
  if (nbody::energy_pair_tasks(n) > INT32_MAX - 8) return NBODY_ERR_INVALID_ARG;
  if (!posmass || !vel || !stats_out) return NBODY_ERR_INVALID_ARG;
  if (!aligned(stats_out, 8)) return NBODY_ERR_ALIGNMENT;
  if (!aligned(posmass, 16) || !aligned(vel, 16)) return NBODY_ERR_ALIGNMENT;
  if (nbody::energy_workspace_bytes(n) > NBODY_ENERGY_STATIC_SCRATCH_BYTES)
    return NBODY_ERR_WORKSPACE;
  const size_t bytes = (size_t)n * 16, sb = 8 * sizeof(double);
  if (overlap(stats_out, sb, posmass, bytes) || overlap(stats_out, sb, vel, bytes))
    return NBODY_ERR_ALIAS;
  void *scratch = nullptr;
  const hipError_t se = nbody::energy_static_scratch(&scratch);
  if (se != hipSuccess) return hip_status(se);
  return hip_status(nbody::launch_energy(posmass, vel, (int)n, G, eps2, scratch, stats_out,
                                         as_stream(stream)));
}

size_t nbody_energy_workspace_bytes(int64_t n) {
  if (!n_ok(n)) return 0;
  return nbody::energy_workspace_bytes(n);
}

int nbody_energy(const float *posmass, const float *vel, int64_t n, float G, float eps2,
                 void *workspace, size_t workspace_bytes, double *stats_out, void *stream) {
  if (!n_ok(n)) return NBODY_ERR_INVALID_ARG;
  if (int s = check_consts(G, eps2)) return s;
  if (n == 0) return NBODY_OK;  // stats_out is left untouched
  if (nbody::energy_pair_tasks(n) > INT32_MAX - 8) return NBODY_ERR_INVALID_ARG;
  if (!posmass || !vel || !stats_out) return NBODY_ERR_INVALID_ARG;
  if (!aligned(stats_out, 8)) return NBODY_ERR_ALIGNMENT;
  if (!aligned(posmass, 16) || !aligned(vel, 16)) return NBODY_ERR_ALIGNMENT;
  const size_t need = nbody::energy_workspace_bytes(n);
  if (!workspace || workspace_bytes < need) return NBODY_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return NBODY_ERR_ALIGNMENT;
  const size_t bytes = (size_t)n * 16, sb = 8 * sizeof(double);
  if (overlap(workspace, need, posmass, bytes) || overlap(workspace, need, vel, bytes) ||
      overlap(workspace, need, stats_out, sb) || overlap(stats_out, sb, posmass, bytes) ||
      overlap(stats_out, sb, vel, bytes))
    return NBODY_ERR_ALIAS;
  return hip_status(nbody::launch_energy(posmass, vel, (int)n, G, eps2, workspace, stats_out,
                                         as_stream(stream)));
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Timing: HIP events recorded on the caller's stream around the timed work.
// ---------------------------------------------------------------------------

struct nbody_timer {
  std::vector<hipEvent_t> ev;
};

namespace {

constexpr int kMaxTimerMarks = 1 << 20;
constexpr int kMaxTimedReps = 1 << 16;

// NBODY_OK when `stream` is not being captured into a graph.
int not_capturing(hipStream_t stream) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  const hipError_t e = hipStreamIsCapturing(stream, &cs);
  if (e != hipSuccess) return hip_status(e);
  return cs == hipStreamCaptureStatusNone ? NBODY_OK : NBODY_ERR_INVALID_ARG;
}

// The force pass of nbody_time_accel and nbody_kdk_run: checks the pass
// kind and that pass's own arguments; *v receives the variant it will run.
int pass_check(const float *posmass, int64_t n, float G, float eps2, const float *accel,
               int pass, int variant, void *workspace, size_t workspace_bytes, int *v) {
  switch (pass) {
    case NBODY_PASS_ONE_SIDED:
      *v = variant < 0 ? nbody::force_variant_for_n(n) : variant;
      return force_aos4_check(posmass, n, G, eps2, accel, *v);
    case NBODY_PASS_SYMMETRIC:
    case NBODY_PASS_SYMMETRIC_POTENTIAL: {
      const bool pot = pass == NBODY_PASS_SYMMETRIC_POTENTIAL;
      *v = sym_variant(variant, n, pot);
      return sym_check(posmass, n, G, eps2, accel, *v, pot, workspace, workspace_bytes, true,
                       true);
    }
    case NBODY_PASS_SYMMETRIC_CHUNKED:
      *v = sym_variant(variant, n, false);
      return sym_check(posmass, n, G, eps2, accel, *v, false, workspace, workspace_bytes, true,
                       true, NBODY_SYMMETRIC_DEFAULT_CHUNK);
    default:
      return NBODY_ERR_INVALID_ARG;
  }
}

void destroy_events(std::vector<hipEvent_t> &ev) {
  for (hipEvent_t &e : ev)
    if (e) (void)hipEventDestroy(e);
  ev.clear();
}

hipError_t create_events(std::vector<hipEvent_t> &ev, int count) {
  ev.assign(count, nullptr);
  for (hipEvent_t &e : ev) {
    const hipError_t r = hipEventCreate(&e);
    if (r != hipSuccess) {
      e = nullptr;
      destroy_events(ev);
      return r;
    }
  }
  return hipSuccess;
}

}  // namespace

extern "C" {

int nbody_timer_create(int marks, nbody_timer **timer_out) {
  if (!timer_out || marks < 1 || marks > kMaxTimerMarks) return NBODY_ERR_INVALID_ARG;
  *timer_out = nullptr;
  nbody_timer *t = new nbody_timer;
  const hipError_t e = create_events(t->ev, marks);
  if (e != hipSuccess) {
    delete t;
    return hip_status(e);
  }
  *timer_out = t;
  return NBODY_OK;
}

int nbody_timer_mark(nbody_timer *timer, int mark, void *stream) {
  if (!timer || mark < 0 || mark >= (int)timer->ev.size()) return NBODY_ERR_INVALID_ARG;
  if (int s = not_capturing(as_stream(stream))) return s;
  return hip_status(hipEventRecord(timer->ev[mark], as_stream(stream)));
}

int nbody_timer_elapsed_ms(nbody_timer *timer, int from, int to, float *ms_out) {
  const int m = timer ? (int)timer->ev.size() : 0;
  if (!timer || !ms_out || from < 0 || from >= m || to < 0 || to >= m)
    return NBODY_ERR_INVALID_ARG;
  hipError_t e = hipEventSynchronize(timer->ev[to]);
  if (e == hipSuccess) e = hipEventElapsedTime(ms_out, timer->ev[from], timer->ev[to]);
  return hip_status(e);
}

int nbody_timer_destroy(nbody_timer *timer) {
  if (!timer) return NBODY_OK;
  destroy_events(timer->ev);
  delete timer;
  return NBODY_OK;
}

int nbody_time_accel(const float *posmass, int64_t n, float G, float eps2, float *accel_out,
                     int pass, int variant, void *workspace, size_t workspace_bytes, int reps,
                     float *pass_ms, float *kernel_ms, void *stream) {
  if (n == 0 || reps < 1 || reps > kMaxTimedReps || !pass_ms) return NBODY_ERR_INVALID_ARG;
  int v;
  if (int s = pass_check(posmass, n, G, eps2, accel_out, pass, variant, workspace,
                         workspace_bytes, &v))
    return s;
  const bool one_sided = pass == NBODY_PASS_ONE_SIDED;
  const bool chunked = pass == NBODY_PASS_SYMMETRIC_CHUNKED;
  const bool pot = pass == NBODY_PASS_SYMMETRIC_POTENTIAL;
  const hipStream_t st = as_stream(stream);
  if (int s = not_capturing(st)) return s;
  // per pass: start, after the dominant kernel, end
  std::vector<hipEvent_t> ev;
  hipError_t e = create_events(ev, 3 * reps);
  BodyArrays b;
  b.posmass = posmass;
  b.accel4 = accel_out;
  for (int r = 0; r < reps && e == hipSuccess; ++r) {
    e = hipEventRecord(ev[3 * r], st);
    if (e == hipSuccess) {
      if (one_sided)
        e = nbody::launch_force(v, Layout::Aos4, b, (int)n, 0, (int)n, G, eps2, st);
      else if (chunked)
        e = nbody::launch_symmetric_chunked(posmass, (int)n, G, eps2, accel_out, v, false,
                                            NBODY_SYMMETRIC_DEFAULT_CHUNK, workspace, st);
      else
        e = nbody::launch_symmetric_tasks(posmass, (int)n, eps2, v, pot, workspace, st);
    }
    if (e == hipSuccess) e = hipEventRecord(ev[3 * r + 1], st);
    if (e == hipSuccess && !one_sided && !chunked)
      e = nbody::launch_symmetric_reduce((int)n, G, accel_out, v, pot, workspace, st);
    if (e == hipSuccess) e = hipEventRecord(ev[3 * r + 2], st);
  }
  if (e == hipSuccess) e = hipEventSynchronize(ev.back());
  for (int r = 0; r < reps && e == hipSuccess; ++r) {
    e = hipEventElapsedTime(&pass_ms[r], ev[3 * r], ev[3 * r + 2]);
    if (e == hipSuccess && kernel_ms)
      e = hipEventElapsedTime(&kernel_ms[r], ev[3 * r], ev[3 * r + 1]);
  }
  destroy_events(ev);
  return hip_status(e);
}

int nbody_kdk_run(float *posmass, float *vel, float *accel, int64_t n, float G, float eps2,
                  float dt, int steps, int pass, int variant, void *workspace,
                  size_t workspace_bytes, void *stream) {
  if (steps < 0 || !isfinite(dt)) return NBODY_ERR_INVALID_ARG;
  int v;
  if (int s = pass_check(posmass, n, G, eps2, accel, pass, variant, workspace, workspace_bytes,
                         &v))
    return s;
  const bool one_sided = pass == NBODY_PASS_ONE_SIDED;
  const bool chunked = pass == NBODY_PASS_SYMMETRIC_CHUNKED;
  const bool pot = pass == NBODY_PASS_SYMMETRIC_POTENTIAL;
  if (n == 0 || steps == 0) return NBODY_OK;
  if (!vel) return NBODY_ERR_INVALID_ARG;
  if (!aligned(vel, 16)) return NBODY_ERR_ALIGNMENT;
  const size_t bytes = (size_t)n * 16;
  if (overlap(vel, bytes, posmass, bytes) || overlap(vel, bytes, accel, bytes) ||
      (!one_sided && overlap(vel, bytes, workspace, workspace_bytes)))
    return NBODY_ERR_ALIAS;
  const hipStream_t st = as_stream(stream);
  // the chunked pass's side stream is shared by every call on the GPU, so a
  // run that uses it is not captured into a caller's graph
  if (chunked)
    if (int s = not_capturing(st)) return s;
  const int ni = (int)n;
  BodyArrays b;
  b.posmass = posmass;
  b.accel4 = accel;
  // step 1 opens with a kick-drift; steps 1 .. steps - 1 end with the force
  // pass and the fused closing kick + next kick-drift; the last step with
  // the force pass and a closing kick
  hipError_t e = nbody::launch_leapfrog(posmass, vel, accel, dt, ni, st);
  for (int s = 1; s <= steps && e == hipSuccess; ++s) {
    if (one_sided)
      e = nbody::launch_force(v, Layout::Aos4, b, ni, 0, ni, G, eps2, st);
    else if (chunked)
      e = nbody::launch_symmetric_chunked(posmass, ni, G, eps2, accel, v, false,
                                          NBODY_SYMMETRIC_DEFAULT_CHUNK, workspace, st);
    else
      e = nbody::launch_symmetric(posmass, ni, G, eps2, accel, v, pot, workspace, st);
    if (e == hipSuccess)
      e = s < steps ? nbody::launch_kick_leapfrog(posmass, vel, accel, dt, ni, st)
                    : nbody::launch_kick(vel, accel, 0.5f * dt, ni, st);
  }
  return hip_status(e);
}

int nbody_set_launch_block_cap(int64_t max_blocks) {
  if (max_blocks < 0) return NBODY_ERR_INVALID_ARG;
  nbody::set_launch_block_cap((long long)max_blocks);
  return NBODY_OK;
}

}  // extern "C"
