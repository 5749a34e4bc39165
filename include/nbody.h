/*
 * nbody.h -- C ABI of libnbody.so: direct all-pairs softened gravity on one
 * AMD Instinct MI355X (gfx950), with a kick-drift-kick leapfrog integrator
 * and a deterministic energy / momentum reduction.
 *
 * The operation (restated from the sources, cited by page and section):
 *   a_i = G * sum_j m_j r_ij / (|r_ij|^2 + eps^2)^{3/2},  r_ij = x_j - x_i,
 * the softened all-pairs acceleration of the "CUDA N-Body Simulation"
 * README (LienoPC/N-BodySimulation), section 1.2, evaluated over float4
 * (x, y, z, m) bodies as in that README's section 2.2 and the tiled kernel of
 * "Cuda Nbody Notes".  The j = i term is included branch-free: r_ii = 0 makes
 * it exactly zero when eps^2 > 0 (README section 1.2, closing remark), which
 * is why eps2 must be > 0.  The host hands positions and masses over and gets
 * accelerations back, the GRAPE-style data flow of the "CAL programming (4)"
 * page (section "N-body computation").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every array pointer is a DEVICE pointer to memory the caller owns (for
 *    instance a torch tensor's data_ptr()).  The library never allocates,
 *    frees, copies to the host or synchronises; every call only enqueues
 *    kernels on `stream` (a hipStream_t passed as void*; NULL = the null
 *    stream) and returns.  Results are ready when the stream reaches them.
 *    The timing calls at the end of this header are the exception: they
 *    create HIP events and wait for them.
 *  - float4 arrays are float[n][4], 16-byte aligned; float3 arrays are
 *    float[n][3] and plain float arrays float[n], 4-byte aligned.
 *  - n is the body count: 0 <= n <= NBODY_MAX_N.  n == 0 is a no-op that
 *    returns NBODY_OK and touches no pointer.
 *  - Arguments are validated before anything is enqueued; on any error
 *    nothing is enqueued.  A failed launch or runtime call returns
 *    NBODY_ERR_HIP, and its error is consumed from HIP's per-thread
 *    last-error state (hipGetLastError), so the caller's next check does not
 *    report it a second time.
 *  - NaN or Inf inside the arrays are not checked; they propagate.
 *  - Outputs are in input order: row i of an output belongs to body i.
 *  - Results are bitwise reproducible for a given (n, entry point, variant):
 *    every sum has a fixed order and no atomics are used.  See
 *    NBODY_SUMMATION_ORDER below.
 *  - The library keeps no state beyond two per-GPU resources made on first
 *    use and kept until the process ends (the side stream and events of
 *    nbody_accel_symmetric_chunked, and the static scratch of
 *    nbody_energy_static) and the process-wide testing cap of
 *    nbody_set_launch_block_cap.  Calls on different streams may overlap as
 *    long as they do not write memory another call reads.
 */
#ifndef NBODY_H
#define NBODY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NBODY_ABI_VERSION 3

/* Largest accepted body count (2^30).  Body indices are 32-bit inside the
 * kernels; byte offsets are 64-bit. */
#define NBODY_MAX_N ((int64_t)1 << 30)

typedef enum nbody_status {
    NBODY_OK = 0,
    NBODY_ERR_INVALID_ARG = -1, /* null pointer with n > 0, n out of range,
                                   eps2 <= 0 or not finite, G / dt not finite,
                                   unknown variant, bad split size */
    NBODY_ERR_ALIGNMENT = -2,   /* a float4 array not 16-byte aligned, or a
                                   float array not 4-byte aligned */
    NBODY_ERR_ALIAS = -3,       /* an output overlaps an array it must not */
    NBODY_ERR_WORKSPACE = -4,   /* workspace NULL or smaller than required */
    NBODY_ERR_HIP = -5          /* a HIP launch or runtime call failed */
} nbody_status;

/* Static, NUL-terminated description of a status code.  Never NULL. */
const char *nbody_status_string(int status);

/* NBODY_ABI_VERSION of the built library. */
int nbody_abi_version(void);

/* ---------------------------------------------------------------------------
 * NBODY_SUMMATION_ORDER (documentation only).
 * For body i, the j range [0, n) is padded to a multiple of the variant's
 * tile width T with bodies of mass 0 (their contribution is exactly +0).  j
 * runs in tiles; inside a tile the three components are accumulated from
 * zero in ascending j with one fused multiply-add per component, and the
 * tile's partial sum is then added to the running sum (two-level summation,
 * which keeps fp32 rounding at ~u*sqrt(n/T) instead of ~u*sqrt(n)).  A
 * variant with LG lane groups keeps LG such sums per body, group g over the
 * tile bodies jj with jj % LG == g (ascending jj), and adds them in
 * ascending g after the last tile.  A variant that splits j over S parts
 * gives each part a contiguous range of tiles and adds the S part sums in
 * ascending part order.  Finally the sum is multiplied by G.
 * ------------------------------------------------------------------------- */

/* Accelerations of all n bodies.
 *   posmass    [n] float4 (x, y, z, m), read only.
 *   G          gravitational constant (finite).
 *   eps2       squared softening length eps^2 (> 0, finite).  The README's
 *              constants table calls this EPS2 (section 6.1).  The pair
 *              terms are fp32: m_j * eps2^(-3/2) must stay below the fp32
 *              maximum (3.4e38) for every body, i.e. eps2 above about
 *              (m_max / 3.4e38)^(2/3) (2e-26 for m = 1, 2e-30 for m = 1e-6).
 *              Below it the self term m_i eps^-3 * 0 is inf * 0 and every
 *              acceleration comes out NaN; this is not checked (the masses
 *              are device data).  The same holds for the split-j passes; the
 *              pair-symmetric passes have a further, mass-independent limit
 *              (see nbody_accel_symmetric).
 *   accel_out  [n] float4, written: (ax, ay, az, 0).  Must not overlap
 *              posmass (NBODY_ERR_ALIAS).
 * The library picks a variant from n (nbody_accel_variant_for_n). */
int nbody_accel(const float *posmass, int64_t n, float G, float eps2,
                float *accel_out, void *stream);

/* The same pass with an explicit compiled variant (0 <= variant <
 * nbody_accel_variant_count()).  For tuning sweeps and tests. */
int nbody_accel_variant(const float *posmass, int64_t n, float G, float eps2,
                        float *accel_out, int variant, void *stream);

/* Number of compiled force variants. */
int nbody_accel_variant_count(void);

/* Describes variant v: bodies per lane, tile width T (the two-level
 * summation chunk), waves per block, j split S, how j-bodies reach the
 * pair step (staging: 0 = LDS tiles, each read serving a whole wavefront
 * or, with lane groups, each lane group from one address; 1 =
 * wave-uniform scalar loads into SGPRs; 2 = vector loads of one address per
 * wavefront, i.e. through the caches only), the unroll factor of the inner
 * j loop (the tunable of the CUDA Handbook's Table 14-2), and the lane
 * groups per wave (LG: lane group g takes the tile's bodies jj with
 * jj % LG == g, and the LG partial sums of a body are added in ascending g
 * after the last tile; 1 = every lane takes every j).  Variants with
 * staging != 0 are an ablation of the LDS design and exist for
 * nbody_accel_variant and nbody_accel_range only.  Returns
 * NBODY_ERR_INVALID_ARG for an unknown v; any pointer may be NULL to skip
 * that field. */
int nbody_accel_variant_info(int v, int *bodies_per_lane, int *tile,
                             int *waves_per_block, int *split, int *staging,
                             int *unroll, int *lane_groups);

/* The variant nbody_accel uses for n bodies. */
int nbody_accel_variant_for_n(int64_t n);

/* nbody_accel plus each body's softened potential in the output's w:
 *   accel_out[i] = (ax, ay, az, Phi_i),
 *   Phi_i = -G sum_{j != i} m_j / sqrt(|x_j - x_i|^2 + eps^2).
 * The CAL IL loop of "CAL programming (4)" carries the same sum in the w
 * lane of its accumulator (its rsq result times m_j).  The j = i pair is
 * dropped from this sum by an index test.  The xyz outputs are bitwise equal
 * to nbody_accel's for the same n.  About three more VALU ops per pair. */
int nbody_accel_potential(const float *posmass, int64_t n, float G, float eps2,
                          float *accel_out, void *stream);

/* Accelerations of bodies [i0, i0 + ni) from all n bodies: the one-sided
 * pass restricted to a contiguous share of the i side, which is what one GPU
 * computes when the pass is split by i ("Cuda Nbody Notes" splits the n
 * bodies into independent blocks of p the same way).
 *   0 <= i0, 0 <= ni, i0 + ni <= n; ni == 0 is a no-op.
 *   accel_out  [ni] float4: row r receives body i0 + r.  Must not overlap
 *              posmass.
 *   variant    a compiled variant, or -1 for nbody_accel_variant_for_n(ni).
 * With the same variant, row r is bitwise equal to row i0 + r of
 * nbody_accel_variant(..., variant): the j side and its order are the same. */
int nbody_accel_range(const float *posmass, int64_t n, int64_t i0, int64_t ni,
                      float G, float eps2, float *accel_out, int variant,
                      void *stream);

/* Two-pass ("2D") decomposition: the j range is cut into chunks of j_chunk
 * bodies (j_chunk a multiple of 32, >= 32); a first kernel writes one
 * float4 partial per (chunk, body) into the workspace, a second adds the
 * chunks of each body in ascending chunk order and multiplies by G.  This
 * is the N x N grid with per-block partial sums and an atomic-free second
 * pass of the README's sections 3.2-3.3, with the chunk as the tunable.
 *   workspace  device memory of at least
 *              nbody_accel_splitj_workspace_bytes(n, j_chunk) bytes, 16-byte
 *              aligned; must not overlap posmass or accel_out.  Contents on
 *              return are unspecified.
 * Other arguments as nbody_accel. */
int nbody_accel_splitj(const float *posmass, int64_t n, float G, float eps2,
                       float *accel_out, int64_t j_chunk, void *workspace,
                       size_t workspace_bytes, void *stream);

/* Workspace bytes nbody_accel_splitj needs (0 for n == 0; 0 for an invalid
 * j_chunk). */
size_t nbody_accel_splitj_workspace_bytes(int64_t n, int64_t j_chunk);

/* Two-pass decomposition with a tree in the first pass (the README's
 * section 3.2 block, and the "first add during load" change of its section
 * 3.4).  A group of X = j_chunk / terms lanes owns one body i and one chunk
 * of j_chunk j-bodies: each lane adds `terms` pair terms in registers (j =
 * c j_chunk + f X + lane, f ascending), then the group halves its width
 * (lane x adds lane x + stride, stride = X/2, ..., 1) and lane 0 writes the
 * chunk's float4 partial; the second pass is nbody_accel_splitj's (chunks in
 * ascending order, times G).  Results are bitwise reproducible for a given
 * (j_chunk, terms) and agree with the other passes to rounding.
 *   terms      1 (plain tree), 2 (FADL) or 4 (fadl4).
 *   j_chunk    terms * X with X one of 8, 16, 32, 64; the README's 32-wide
 *              block is j_chunk = 32 with X = 32, 16, 8 for terms 1, 2, 4.
 *              The chunk count ceil(n / j_chunk) must be <= 65535.
 *   workspace  >= nbody_accel_splitj_tree_workspace_bytes(n, j_chunk, terms)
 *              bytes (ceil(n / j_chunk) * n float4), 16-byte aligned,
 *              disjoint from posmass and accel_out; contents on return are
 *              unspecified.
 * Other arguments as nbody_accel; NBODY_ERR_INVALID_ARG for any other
 * (j_chunk, terms). */
int nbody_accel_splitj_tree(const float *posmass, int64_t n, float G, float eps2,
                            float *accel_out, int64_t j_chunk, int terms, void *workspace,
                            size_t workspace_bytes, void *stream);

/* Workspace bytes nbody_accel_splitj_tree needs (0 for n == 0 or an invalid
 * (j_chunk, terms)). */
size_t nbody_accel_splitj_tree_workspace_bytes(int64_t n, int64_t j_chunk, int terms);

/* Pair-symmetric force pass: each unordered pair is evaluated once and its
 * term is applied to both bodies (Newton's third law).  The atomics tutorial
 * ("CUDA programming (9)", neighbour-list example) runs this symmetric half
 * loop with atomicAdd for the second body; here no atomics are used: the
 * second body's share is carried either in registers rotated across the
 * wavefront or in a per-wave LDS slot that one lane at a time reads, adds to
 * and writes back, and every sum has a fixed order, so the result is bitwise
 * reproducible for a given (n, variant).  Bodies are grouped in
 * panels of nbody_accel_symmetric_panel(variant) bodies; a panel pair (I, J)
 * writes panel I's sums from J and panel J's sums from I into the
 * workspace, and a second kernel adds, for each body, the P panel sums in
 * blocks of 32 panels (each block's sums in ascending panel order into a
 * fresh block sum, the block sums in ascending order) and multiplies by G.
 * The order differs from
 * nbody_accel's, so the two agree to rounding, not bitwise; variants that
 * carry the second body's share differently (registers or LDS) also agree
 * to rounding only.
 *   variant    0 <= variant < nbody_accel_symmetric_variant_count(), or -1
 *              for the library's choice.
 *   workspace  >= nbody_accel_symmetric_workspace_bytes(n, variant) bytes
 *              (12 n^2 / panel bytes: about 6.4 GB at n = 2^20), 16-byte
 *              aligned, disjoint from posmass and accel_out; contents on
 *              return are unspecified.
 * eps2 range: a pair in two different panels forms inv^3 = (|r|^2 +
 * eps^2)^(-3/2) in fp32 before either mass multiplies it (one product serves
 * both bodies), so besides nbody_accel's limit eps2 must stay above about
 * 2.1e-26 whatever the masses: below it inv^3 overflows for coincident
 * bodies in different panels, and both their rows come out NaN (inf * 0).
 * A diagonal panel pair (I, I) keeps nbody_accel's mass-first form, so
 * coincident bodies in one panel follow nbody_accel's limit: in the 4-wave
 * variants (0, 1, 4) it is summed one-sidedly, j = i included; in the
 * one-wave variants (2, 3) each pair of the panel is met once and j = i is
 * never formed, so the self term, and its overflow, do not arise.  Not
 * checked.
 * Other arguments as nbody_accel.  NBODY_ERR_INVALID_ARG also when the
 * panel pairs exceed 2^31 - 1 (n beyond ~1.3e8). */
int nbody_accel_symmetric(const float *posmass, int64_t n, float G, float eps2,
                          float *accel_out, int variant, void *workspace,
                          size_t workspace_bytes, void *stream);
/* Workspace bytes for (n, variant); variant -1 means the library's choice
 * for n.  0 for n == 0 or an unknown variant. */
size_t nbody_accel_symmetric_workspace_bytes(int64_t n, int variant);
/* Number of compiled variants of the pair-symmetric pass. */
int nbody_accel_symmetric_variant_count(void);
/* Panel size (bodies) of a variant; NBODY_ERR_INVALID_ARG if unknown. */
int nbody_accel_symmetric_panel(int variant);
/* The variant nbody_accel_symmetric uses for n when passed -1. */
int nbody_accel_symmetric_variant_for_n(int64_t n);

/* nbody_accel_symmetric in column chunks, with a workspace that grows as n,
 * not n^2.  The panel pairs (I, J) are taken chunk by chunk, a chunk being
 * the pairs with J in a range of chunk_panels panels (ascending ranges);
 * after each chunk's panel-pair kernel, a reduce kernel adds that chunk's
 * panel sums into each touched body's fp32 running sum (kept in accel_out
 * between chunks) in the same blocks of 32 panels, ascending (chunk bounds
 * are multiples of 32), and the last chunk multiplies by G.  Each body's
 * panel sums are therefore added in the same order as by
 * nbody_accel_symmetric, and accel_out is bitwise equal to its result for
 * the same variant, whatever chunk_panels.
 * Consecutive chunks run on two queues, in two halves of the workspace:
 * even chunks on `stream`, odd chunks on a side stream the library creates
 * for the current GPU on first use (default priority, kept until the
 * process ends, with a pool of events), so that one chunk's panel-pair
 * kernel fills the CUs the previous one's tail leaves idle.  The calls are
 * ordered by events: the call is asynchronous on `stream` like every entry
 * point, and work queued on `stream` after it starts only when the whole
 * pass is done.  Calls on one GPU share the side stream (they are correct
 * but serialise there); the stream must belong to the current HIP device.
 *   chunk_panels  a positive multiple of 32 (the panel-pair tile side), or 0
 *                 for NBODY_SYMMETRIC_DEFAULT_CHUNK.
 *   workspace     >= nbody_accel_symmetric_chunked_workspace_bytes(n,
 *                 variant, chunk_panels) bytes: two chunks' panel sums,
 *                 about 48 n chunk_panels bytes (1.6 GB at n = 2^20 with
 *                 32, against 6.4 GB for nbody_accel_symmetric; 9 GB at
 *                 6e6 bodies, where the whole pass would need 211 GB).
 *                 16-byte aligned, disjoint from posmass and accel_out;
 *                 contents on return are unspecified.
 * Two launches per chunk; other arguments and errors as
 * nbody_accel_symmetric (NBODY_ERR_INVALID_ARG for a bad chunk_panels). */
#define NBODY_SYMMETRIC_DEFAULT_CHUNK 32
int nbody_accel_symmetric_chunked(const float *posmass, int64_t n, float G, float eps2,
                                  float *accel_out, int variant, int chunk_panels,
                                  void *workspace, size_t workspace_bytes, void *stream);
/* Workspace bytes for (n, variant, chunk_panels); 0 for n == 0, an unknown
 * variant or a bad chunk_panels. */
size_t nbody_accel_symmetric_chunked_workspace_bytes(int64_t n, int variant, int chunk_panels);

/* nbody_accel_symmetric in its two phases, for callers that schedule them
 * themselves (other work between them, or timing the panel-pair kernel on
 * its own).  nbody_accel_symmetric_tasks runs the panel-pair kernel: it reads
 * posmass and writes every panel sum into the workspace.
 * nbody_accel_symmetric_reduce runs the second kernel: it adds each body's
 * panel sums (blocks of 32 panels, ascending) into accel_out, times G.  The reduce
 * must be given the same n, variant and workspace, with the contents the
 * tasks call left, on the same stream or one ordered after it; the pair
 * then gives accel_out bitwise equal to nbody_accel_symmetric's.  Arguments,
 * workspace size and errors as nbody_accel_symmetric, restricted to the
 * arrays each phase touches (the tasks phase checks eps2, the reduce G). */
int nbody_accel_symmetric_tasks(const float *posmass, int64_t n, float eps2, int variant,
                                void *workspace, size_t workspace_bytes, void *stream);
int nbody_accel_symmetric_reduce(int64_t n, float G, float *accel_out, int variant,
                                 const void *workspace, size_t workspace_bytes, void *stream);

/* The pair-symmetric pass that also carries each body's potential, as
 * nbody_accel_potential does for the one-sided pass (the CAL IL loop of "CAL
 * programming (4)" keeps the same sum, m_j times its rsq result, in the w
 * lane of its accumulator):
 *   accel_out[i] = (ax, ay, az, Phi_i),
 *   Phi_i = -G sum_{j != i} m_j / sqrt(|x_j - x_i|^2 + eps^2).
 * Each unordered pair adds m_j inv to body i's sum and m_i inv to body j's
 * (two more multiply-adds per pair); the j = i pair is left out (by an
 * index test in the one-sided diagonal panel pairs of the 4-wave variants;
 * the one-wave variants never form it).  The potential sums follow the
 * acceleration's order (per panel pair, then panel pairs in ascending
 * order).  Its variants are a table of their own (ids below).  The xyz
 * outputs are bitwise equal to nbody_accel_symmetric's for a variant of the
 * same panel shape; the default choices (variant -1 on both) have the same
 * shape at every n.  With
 * nbody_energy_from_potential this gives the energy of a checkpoint step
 * without a separate pair pass.
 *   workspace  >= nbody_accel_symmetric_potential_workspace_bytes(n, variant)
 *              bytes (16 n^2 / panel bytes), 16-byte aligned, disjoint from
 *              posmass and accel_out; contents on return are unspecified.
 * Other arguments and errors as nbody_accel_symmetric. */
int nbody_accel_symmetric_potential(const float *posmass, int64_t n, float G, float eps2,
                                    float *accel_out, int variant, void *workspace,
                                    size_t workspace_bytes, void *stream);
size_t nbody_accel_symmetric_potential_workspace_bytes(int64_t n, int variant);
int nbody_accel_symmetric_potential_variant_count(void);
int nbody_accel_symmetric_potential_panel(int variant);
int nbody_accel_symmetric_potential_variant_for_n(int64_t n);

/* The force pass on other body layouts; same arithmetic and order as
 * nbody_accel for the same n, so the outputs are bitwise equal to its
 * (ax, ay, az).  README section 3.5 compares float4 against 12-byte float3
 * records.
 *   nbody_accel_f3aos: pos [n] float3 (x, y, z), mass [n] float,
 *                      accel_out [n] float3 (ax, ay, az).
 *   nbody_accel_soa:   x, y, z, m, ax, ay, az: [n] float each.
 * No output may overlap an input. */
int nbody_accel_f3aos(const float *pos, const float *mass, int64_t n, float G,
                      float eps2, float *accel_out, void *stream);
int nbody_accel_soa(const float *x, const float *y, const float *z,
                    const float *m, int64_t n, float G, float eps2, float *ax,
                    float *ay, float *az, void *stream);

/* Kick and drift of the leapfrog scheme, README section 1.3:
 *   v <- v + (dt/2) a ;  x <- x + dt v   (per body, in place)
 *   posmass  [n] float4, xyz updated, m (w) left bit-for-bit unchanged.
 *   vel      [n] float4, xyz updated, w left unchanged.
 *   accel    [n] float4, a(x) at the current positions (w ignored).
 * The three arrays must be pairwise disjoint.  A full kick-drift-kick step
 * is nbody_leapfrog_step, nbody_accel at the new positions, then
 * nbody_kick(vel, accel, dt/2). */
int nbody_leapfrog_step(float *posmass, float *vel, const float *accel,
                        float dt, int64_t n, void *stream);

/* Closing half-kick v <- v + h a (h = dt/2 for kick-drift-kick).  The
 * README's section 1.3 prints one half kick and a drift per step and keeps
 * the velocities at half steps; this library reads the scheme as standard
 * kick-drift-kick leapfrog, so that the velocities are synchronised with
 * the positions after every step (and energy is defined there): the step is
 * nbody_leapfrog_step (the printed two updates), a force pass at the new
 * positions, then this second half kick with the new accelerations.
 *   vel [n] float4 in place (w unchanged); accel [n] float4, disjoint. */
int nbody_kick(float *vel, const float *accel, float h, int64_t n,
               void *stream);

/* `steps` kick-drift-kick steps (README section 1.3, read as above: the
 * printed kick and drift, a force pass, the closing half kick) run by the
 * library: exactly nbody_leapfrog_step, the force pass and nbody_kick with
 * h = dt/2, step after step, except that the closing half kick of a step and
 * the kick-drift of the next, which use the same accelerations, run as one
 * kernel doing the same operations in the same order.  The result is
 * bitwise that of the calls made one by one.
 *   posmass, vel  [n] float4, in place (masses and vel.w unchanged).
 *   accel         [n] float4: on entry the accelerations at the current
 *                 positions (for example from a force pass); on return those
 *                 at the final positions.  With NBODY_PASS_SYMMETRIC_POTENTIAL
 *                 accel.w carries Phi_i on return (it is not read).
 *   pass          one of the NBODY_PASS_* values defined with
 *                 nbody_time_accel below: the one-sided pass
 *                 (nbody_accel_variant), the pair-symmetric pass, that pass
 *                 with the potential, or the pair-symmetric pass in column
 *                 chunks of NBODY_SYMMETRIC_DEFAULT_CHUNK panels (bitwise
 *                 the whole pass's result, in a workspace of about 48 n 32
 *                 bytes); variant -1 for the library's choice; workspace as
 *                 that pass needs (unused by the one-sided pass).
 * Like every compute entry point it allocates nothing and does not
 * synchronise, and it records no memset, so a caller may capture it into a
 * HIP graph on a stream of its own and replay it; with
 * NBODY_PASS_SYMMETRIC_CHUNKED, whose side stream every call on the GPU
 * shares, a stream being captured is NBODY_ERR_INVALID_ARG instead.
 * steps == 0 or n == 0 is a no-op.  The arrays must be pairwise disjoint
 * and disjoint from the workspace.  Other arguments and errors as the force
 * pass and nbody_leapfrog_step. */
int nbody_kdk_run(float *posmass, float *vel, float *accel, int64_t n, float G, float eps2,
                  float dt, int steps, int pass, int variant, void *workspace,
                  size_t workspace_bytes, void *stream);

/* Energy and momentum.  stats_out (device, 8 doubles) receives
 *   {K, W, K + W, Px, Py, Pz, M, 0}
 * with K = sum m |v|^2 / 2, P = sum m v, M = sum m and
 * W = -G sum_{i<j} m_i m_j / sqrt(|x_i - x_j|^2 + eps^2), the softened
 * potential whose negative gradient is the acceleration above (the pages
 * print no energy; this is the plain reading).  W is summed over panel pairs
 * with every unordered pair met once (as in nbody_accel_symmetric): pair
 * terms in fp32 over 64-body sweeps, then fp64, and every cross-lane,
 * cross-task and cross-body sum in a fixed fp64 tree order.  n above about
 * 1.3e8 (more than 2^31 - 1 panel pairs) is NBODY_ERR_INVALID_ARG.
 *   workspace  >= nbody_energy_workspace_bytes(n) bytes, 16-byte aligned,
 *              disjoint from every other argument.
 *   stats_out  8 doubles, 8-byte aligned. */
int nbody_energy(const float *posmass, const float *vel, int64_t n, float G,
                 float eps2, void *workspace, size_t workspace_bytes,
                 double *stats_out, void *stream);

size_t nbody_energy_workspace_bytes(int64_t n);

/* nbody_energy without a caller workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving or simulation
 * loops, harnesses that forbid hipMalloc.  The same kernels and the same
 * fixed summation order as nbody_energy, so stats_out is bitwise equal to
 * nbody_energy's for the same inputs.  Their scratch (per-block and per
 * panel-pair fp64 partial sums, nbody_energy_workspace_bytes(n) bytes) is a
 * static device array of NBODY_ENERGY_STATIC_SCRATCH_BYTES inside the
 * library, one per GPU, held until the process ends; its device address is
 * looked up once per GPU, on the first call made with that GPU current.
 * Nothing in it needs to start at zero: every call writes each partial it
 * reads.  The call allocates nothing and frees nothing.
 *   n          0 <= n, with nbody_energy_workspace_bytes(n) <=
 *              NBODY_ENERGY_STATIC_SCRATCH_BYTES, i.e. n <= 4,063,232;
 *              larger n is NBODY_ERR_WORKSPACE.
 *   stream     must belong to the current HIP device.
 * Every call on one GPU shares that GPU's scratch: calls that overlap on one
 * GPU (on different streams, or from different host threads) race on it and
 * must be ordered by the caller.  Other arguments and errors as
 * nbody_energy. */
#define NBODY_ENERGY_STATIC_SCRATCH_BYTES ((size_t)16 << 20)
int nbody_energy_static(const float *posmass, const float *vel, int64_t n, float G,
                        float eps2, double *stats_out, void *stream);

/* Energy and momentum in O(n) from the potentials nbody_accel_potential or
 * nbody_accel_symmetric_potential stored in accel_pot[i].w: stats_out = {K, W, K + W, Px, Py, Pz, M, 0}
 * with W = sum_i m_i Phi_i / 2 (each pair once).  fp64 fixed-order
 * reduction as in nbody_energy.
 *   workspace  >= nbody_energy_from_potential_workspace_bytes(n) bytes,
 *              16-byte aligned, disjoint from every other argument. */
int nbody_energy_from_potential(const float *posmass, const float *vel,
                                const float *accel_pot, int64_t n,
                                void *workspace, size_t workspace_bytes,
                                double *stats_out, void *stream);
size_t nbody_energy_from_potential_workspace_bytes(int64_t n);

/* ---------------------------------------------------------------------------
 * Timing, for benchmarks.  HIP events created by the library and recorded
 * on the stream the timed work is launched on: the event-timing pattern of
 * the atomics tutorial ("CUDA programming (9)", its timing() helper: record
 * an event, run the work, record a second event, wait for it, read the
 * elapsed time), repeated over several runs.  These calls, unlike the rest
 * of the library, create and destroy HIP events, and nbody_time_accel and
 * nbody_timer_elapsed_ms wait for the GPU; none of them may be used while
 * the stream is being captured into a graph (NBODY_ERR_INVALID_ARG).  The
 * stream must belong to the current HIP device.
 * ------------------------------------------------------------------------- */

/* An opaque set of HIP events ("marks") for bracketing work on streams. */
typedef struct nbody_timer nbody_timer;

/* Creates a timer of `marks` events (1 <= marks <= 1 << 20). */
int nbody_timer_create(int marks, nbody_timer **timer_out);
/* Records event `mark` on `stream` (a later call re-records it). */
int nbody_timer_mark(nbody_timer *timer, int mark, void *stream);
/* Waits for event `to` and writes the time from event `from` to event `to`
 * in milliseconds.  NBODY_ERR_HIP if either was never recorded. */
int nbody_timer_elapsed_ms(nbody_timer *timer, int from, int to, float *ms_out);
/* Destroys the timer's events and frees it (NULL is a no-op). */
int nbody_timer_destroy(nbody_timer *timer);

/* Force passes nbody_time_accel can run. */
#define NBODY_PASS_ONE_SIDED 0            /* nbody_accel_variant; -1: nbody_accel */
#define NBODY_PASS_SYMMETRIC 1            /* nbody_accel_symmetric */
#define NBODY_PASS_SYMMETRIC_POTENTIAL 2  /* nbody_accel_symmetric_potential */
#define NBODY_PASS_SYMMETRIC_CHUNKED 3    /* nbody_accel_symmetric_chunked, default chunk */

/* Runs `reps` force passes of the given kind back to back on `stream`, each
 * bracketed by events recorded inside the library, waits for the last, and
 * writes the host arrays:
 *   pass_ms[r]    duration of pass r (all of its kernels);
 *   kernel_ms[r]  duration of its dominant kernel alone: the panel-pair
 *                 kernel of the pair-symmetric passes (their reduce kernel
 *                 follows it), the whole pass for the one-sided one and for
 *                 the chunked one (whose chunks overlap on two queues).  May
 *                 be NULL.
 *   variant       as the pass's entry point (-1: the library's choice).
 *   workspace     the pair-symmetric passes' workspace (ignored for the
 *                 one-sided pass; may then be NULL); for the chunked pass
 *                 nbody_accel_symmetric_chunked_workspace_bytes(n, variant,
 *                 0) bytes.
 * Other arguments, sizes and errors as the pass's entry point; additionally
 * NBODY_ERR_INVALID_ARG for n == 0, reps < 1 or reps > 1 << 16, an unknown
 * pass, a NULL pass_ms, or a stream being captured. */
int nbody_time_accel(const float *posmass, int64_t n, float G, float eps2,
                     float *accel_out, int pass, int variant, void *workspace,
                     size_t workspace_bytes, int reps, float *pass_ms,
                     float *kernel_ms, void *stream);

/* ---------------------------------------------------------------------------
 * Launch splitting.  HIP counts a launch's size in work-items with 32 bits
 * per grid dimension.  The passes whose grid can outgrow that (the one-sided
 * pass, 16 or 32 threads per body; the pair-symmetric and energy passes, one
 * block per panel pair: from about 1.2e7 bodies for the energy) issue their
 * blocks in several launches of at most (2^32 - 1) / block-threads blocks.
 * Every block computes the same thing in any launch, so results are bitwise
 * those of one launch.
 *
 * nbody_set_launch_block_cap lowers that per-launch block count to
 * max_blocks for every later call in the process (0 restores the hardware
 * limit), so that small inputs take the split path too: a testing aid, not
 * a tuning knob.  It is a process-wide setting read at each launch; calls
 * already enqueued are unaffected.  Returns NBODY_ERR_INVALID_ARG for
 * max_blocks < 0.
 * ------------------------------------------------------------------------- */
int nbody_set_launch_block_cap(int64_t max_blocks);

#ifdef __cplusplus
}
#endif

#endif /* NBODY_H */
