/*
 * schnet_mi355x.h - C ABI of the SchNet continuous-filter convolution (CFConv)
 * energy and force library for AMD Instinct MI355X (gfx950).
 *
 * The operations are those of "FlashSchNet: Fast and Accurate Coarse-Grained
 * Neural Network Molecular Dynamics" (arXiv 2602.13140): the neighbour list of
 * §3.2 "Building the neighbor list" grouped by destination as in §4.3 "Index
 * construction under dynamic neighbor lists"; the energy of §3.2 "SchNet model"
 * (distances, radial basis with cosine envelope, filter network, CFConv
 * aggregation, update network, readout) evaluated as in §4.2 "Fused forward
 * operator" and §4.3 "Destination grouped segmented reduction"; forces
 * F = -dE/dr (§3.1, §3.2 "Forces via autodiff"); and the Langevin MD step over
 * parallel replicas of §4.5 "End-to-end integration" and §5.1.
 *
 * Conventions for every call:
 *  - Pointers are DEVICE pointers unless the argument name ends in _host.
 *    The caller allocates and owns every buffer; the library allocates device
 *    memory only in sn_model_create (its own weight copy).
 *  - Work is enqueued on the caller's stream and returns without waiting,
 *    except where a call says it synchronises.
 *  - Arguments are validated on the host before anything is launched; an
 *    invalid argument returns SN_ERR_INVALID_ARG and enqueues nothing.
 *  - Errors found on the device (list capacity, non-finite energies,
 *    positions or velocities, atom types out of range, lists too long) are
 *    recorded in a status word inside the workspace; read it with
 *    sn_get_device_status. The first error wins until sn_reset_device_status.
 *  - Atoms are numbered replica-major: atom a of replica r is r*N + a, with
 *    N = atoms_per_replica. Positions and forces are float [R*N][3].
 *  - Units: Angstrom, kcal/mol, amu, fs, K.
 *  - A model handle is immutable after creation and may be shared by streams;
 *    a workspace belongs to one stream at a time.
 */
#ifndef SCHNET_MI355X_H
#define SCHNET_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t; /* HIP stream handle; NULL = default stream */

typedef enum {
  SN_OK = 0,
  SN_ERR_INVALID_ARG = 1,  /* bad pointer, size, shape or geometry */
  SN_ERR_CAPACITY = 2,     /* the neighbour list needs more than edge_capacity slots */
  SN_ERR_NONFINITE = 3,    /* a replica energy, a position given to a neighbour
                              build or an MD position or velocity is NaN or infinite */
  SN_ERR_UNSUPPORTED = 4,  /* a model or system shape this build does not handle */
  SN_ERR_HIP = 5,          /* a HIP runtime call failed */
  SN_ERR_WORKSPACE = 6     /* the workspace is smaller than sn_workspace_size says */
} sn_status;

/* Operand precision of the networks (sn_model_desc.filter_dtype):
 *  SN_FILTER_F32   every product in fp32;
 *  SN_FILTER_BF16  the filter network's products take bfloat16 operands
 *                  (weights rounded to nearest even, activations rounded as
 *                  they enter a product); the update and readout layers
 *                  keep fp32-grade products on fp16 pairs, as
 *                  SN_FILTER_F16X2 describes (in the fused calls and in the
 *                  unfused pipeline alike);
 *  SN_W16A16       every MLP (filter, update, readout) takes fp16 operands,
 *                  with per-output-channel scales (§4.4 "Channel-wise
 *                  quantization"): each weight column n is stored as
 *                  fp16(W[:, n] / s_n) with s_n the power of two at or above
 *                  the column's largest magnitude (1 for a zero column), and
 *                  the readout's output weights likewise as one column;
 *  SN_FILTER_F16X2 the fp32 model with every MLP product (filter, update,
 *                  readout) on the fp16 matrix units: each fp32 weight and
 *                  activation enters as a pair of fp16 numbers hi + lo (22
 *                  significant bits) after a power-of-two scaling that keeps
 *                  both parts in fp16's normal range (per matrix; per
 *                  filter input from bounds derived on the host from the
 *                  weights and the basis width; per atom for the update and
 *                  readout inputs), and each product is hi*hi + hi*lo +
 *                  lo*hi: about 1e-6 relative error per dot product, inside
 *                  the fp32 tolerances. The energy+force and MD calls accept
 *                  it; the unfused pipeline returns SN_ERR_UNSUPPORTED.
 * Accumulation is fp32 in every case; positions, distances, basis
 * functions, biases, energies and forces stay fp32. */
enum { SN_FILTER_F32 = 0, SN_FILTER_BF16 = 1, SN_W16A16 = 2, SN_FILTER_F16X2 = 3 };

/* Model shape. Supported: D in {64, 128}; 2 <= Dr <= 64; 1 <= T <= 8;
 * H in {32, 64} with H <= D; n_types >= 1; 0 <= rbf_min < rbf_max;
 * r_cut > 0; filter_dtype one of the precisions above. */
typedef struct {
  int32_t n_types;   /* number of atom/bead types */
  int32_t D;         /* hidden feature width */
  int32_t Dr;        /* number of Gaussian radial basis functions */
  int32_t T;         /* number of interaction blocks */
  int32_t H;         /* readout hidden width */
  float rbf_min;     /* first Gaussian centre */
  float rbf_max;     /* last Gaussian centre; width = spacing of centres */
  float r_cut;       /* cosine-envelope cutoff; listed edges at or beyond it contribute 0 */
  int32_t filter_dtype;
} sn_model_desc;

/* R independent replicas of N atoms each. periodic != 0 makes every replica a
 * cube of side `box` with minimum-image distances; positions must then lie in
 * [0, box). Edges never join two replicas. */
typedef struct {
  int32_t n_replicas;
  int32_t atoms_per_replica;
  int32_t periodic;
  float box;
} sn_system;

typedef struct sn_model sn_model;

/* Number of floats in the flat weight vector for `desc`, 0 if desc is invalid.
 * Layout (row-major [fan_in][fan_out] matrices):
 *   Emb[n_types][D];
 *   for each block t: Wf1[Dr][D], cf1[D], Wf2[D][D], cf2[D],
 *                     Wu1[D][D], cu1[D], Wu2[D][D], cu2[D];
 *   Wo1[D][H], co1[H], Wo2[H], co2[1].
 * Block t computes  w_e = ssp(b_e Wf1 + cf1) Wf2 + cf2  (filter, §3.2 "Filter
 * network"),  h_i = sum_{dst(e)=i} x_src(e) * w_e  (CFConv), and
 * x' = x + ssp(h Wu1 + cu1) Wu2 + cu2  (update with residual); the readout is
 * eps_i = ssp(x_i Wo1 + co1) . Wo2 + co2 and E_r = sum of eps_i over replica r.
 * ssp(z) = ln(1 + e^z) - ln 2. */
size_t sn_model_weight_count(const sn_model_desc* desc);

/* Validates desc, copies `n_floats` host floats to the device (converting the
 * network matrices to the 16-bit formats filter_dtype selects) and returns
 * a handle in *out. Synchronises the current device. Errors:
 * SN_ERR_INVALID_ARG (null pointers, n_floats mismatch), SN_ERR_UNSUPPORTED
 * (shape outside the supported set), SN_ERR_HIP. */
sn_status sn_model_create(const sn_model_desc* desc, const float* weights_host, size_t n_floats,
                          sn_model** out);
void sn_model_destroy(sn_model* model);

/* Bytes of device workspace that sn_build_neighbors, sn_energy_forces and the
 * MD calls need for `sys` and a model of shape `desc` (desc may be NULL when
 * only the neighbour list is built). The workspace carries intermediate
 * per-atom arrays, neighbour-build scratch and the device status word; nothing
 * edge-sized is ever stored in it. Clear it once with sn_reset_device_status
 * after allocating it. */
sn_status sn_workspace_size(const sn_model_desc* desc, const sn_system* sys, size_t* bytes_host);

/* Directed neighbour list within r_list, grouped by receiver (CSR).
 * Edge j -> i exists iff i != j, both lie in the same replica and
 * s < r*r, where, in IEEE double arithmetic without contraction on the float
 * inputs, delta = x_j - x_i per axis (minimum image for a periodic cube:
 * delta -= L if delta > L/2, delta += L if delta < -L/2) and
 * s = (dx*dx + dy*dy) + dz*dz, r being the double value of r_list.
 * Output: rowptr[R*N + 1] (int32) and col[edge_capacity] (int32); receiver i
 * owns col[rowptr[i] .. rowptr[i+1]), senders ascending. The list is therefore
 * symmetric. Periodic systems need box >= 2*r_list.
 * If the list needs more than edge_capacity slots, the device status becomes
 * SN_ERR_CAPACITY with the needed count as detail, every row of rowptr is left
 * empty and col is not written. If n_edges_host is not NULL the call
 * synchronises the stream and stores the edge count there (also on overflow).
 * Positions must be finite: a NaN or infinite coordinate of atom i sets the
 * device status to SN_ERR_NONFINITE with detail -(1 + i) (such an atom
 * would otherwise pass no membership test and silently lose its edges). */
sn_status sn_build_neighbors(const sn_system* sys, const float* pos, float r_list, int32_t* rowptr,
                             int32_t* col, int64_t edge_capacity, int64_t* n_edges_host, void* ws,
                             size_t ws_bytes, hipStream_t stream);

/* Energies energy[R] and forces forces[R*N][3] = -dE/dr for positions pos and
 * types[R*N] (int32 in [0, n_types)), on a list from sn_build_neighbors built
 * with r_list >= r_cut (a larger radius, for instance with a skin, is allowed).
 * The list must be symmetric, as that call makes it: the force on atom i is
 * gathered from i's own row. fp32 inputs and outputs, fp32 accumulation.
 * A list of 2^30 or more edges sets the device status to SN_ERR_UNSUPPORTED
 * (detail: the edge count) and leaves the outputs invalid; a type outside
 * [0, n_types) sets it to SN_ERR_INVALID_ARG (detail: an offending atom), is
 * read as type 0, and leaves the outputs invalid. */
sn_status sn_energy_forces(const sn_model* model, const sn_system* sys, const float* pos,
                           const int32_t* types, const int32_t* rowptr, const int32_t* col,
                           float* energy, float* forces, void* ws, size_t ws_bytes,
                           hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the
 * energies and forces of sn_energy_forces, same arguments and results, with
 * the workspace taken from a static device array of the library instead of
 * a caller's buffer. The call allocates nothing. The array holds
 * SN_SCRATCH_BYTES (32 MiB) on each GPU the library runs on, until the
 * process ends; a system whose workspace (sn_workspace_size) is larger is
 * refused with SN_ERR_WORKSPACE before anything is enqueued (at D = 128,
 * T = 3 that is above about 5,000 atoms; the 4096-atom box fits).
 * The array's status block is cleared at the start of every call, and when
 * the call's work completes its sn_status and detail (as
 * sn_get_device_status reports them) are written to status_dev[0] and
 * status_dev[1] (device memory, int64). Every call on a GPU shares that
 * GPU's array, which keeps the last call's contents: calls on one stream are
 * ordered and safe, calls that overlap on one GPU (other streams, other
 * threads) race and give wrong results. No profiling events are recorded. */
#define SN_SCRATCH_BYTES ((size_t)32 << 20)
sn_status sn_energy_forces_noalloc(const sn_model* model, const sn_system* sys, const float* pos,
                                   const int32_t* types, const int32_t* rowptr,
                                   const int32_t* col, float* energy, float* forces,
                                   int64_t* status_dev, hipStream_t stream);

/* The same energies and forces by the unfused pipeline that FlashSchNet
 * measures its techniques against (§3.3 bottlenecks, Fig. 2(b) lower
 * pipeline; §4.5 "End-to-end integration" names fusion and segmented
 * reduction as ablation switches), so that both can be timed on one GPU.
 * Each step of the edge path is a separate kernel whose output is an edge
 * tensor in the workspace: distances, Gaussians, envelope, basis B[E][Dr],
 * filter pre-activation, activation and filter W[E][D], gathered sender rows
 * X_src[E][D] and messages M[E][D]; the backward applies the chain rule
 * through the same tensors. Aggregation (messages into receivers, feature
 * gradients into senders, dE/dr into both ends of each edge) is a segment sum
 * over the receiver rows, the sender side through the reverse-edge index of
 * the symmetric list, or with flags = SN_UNFUSED_ATOMIC atomic adds; atomic
 * results are not bitwise reproducible. The embedding, update and readout
 * layers are the ones sn_energy_forces runs.
 * edge_capacity (>= 1) bounds the list's edge count rowptr[R*N]: every edge
 * tensor has that many rows. A larger list sets the device status to
 * SN_ERR_CAPACITY and leaves the outputs invalid. Other arguments as for
 * sn_energy_forces; the list must come from sn_build_neighbors (symmetric,
 * senders ascending). Models with filter_dtype SN_W16A16 or SN_FILTER_F16X2
 * return SN_ERR_UNSUPPORTED. */
enum { SN_UNFUSED_ATOMIC = 1 };

/* Workspace bytes for sn_energy_forces_unfused: the sn_workspace_size amount
 * plus about 4 (3T + 4) D + 8 Dr edge-tensor bytes per edge of capacity. */
sn_status sn_unfused_workspace_size(const sn_model_desc* desc, const sn_system* sys,
                                    int64_t edge_capacity, size_t* bytes_host);
sn_status sn_energy_forces_unfused(const sn_model* model, const sn_system* sys, const float* pos,
                                   const int32_t* types, const int32_t* rowptr,
                                   const int32_t* col, int64_t edge_capacity, int32_t flags,
                                   float* energy, float* forces, void* ws, size_t ws_bytes,
                                   hipStream_t stream);

/* Langevin dynamics by BAOAB splitting:
 *   v += dt/2 k F/m;  r += dt/2 v;  v = c1 v + c2 xi;  r += dt/2 v;
 *   (rebuild list if due);  F = F(r);  v += dt/2 k F/m
 * with c1 = exp(-gamma dt), c2 = sqrt((1 - c1^2) kB T k / m),
 * k = 4.184e-4 A/fs^2 per kcal/mol/A/amu, kB = 0.0019872043 kcal/mol/K.
 * xi: standard normals from Philox4x64-10 keyed (seed, 0) with counter
 * (global atom, step, 0, 0); the four words become uniforms
 * ((w >> 11) + 0.5) 2^-53 and Box-Muller on (u0, u1), (u2, u3) gives the
 * x, y and z components (the fourth normal is unused). */
typedef struct {
  float dt_fs;
  float temperature_K;
  float gamma_per_ps;
  float mass_amu;
  float skin;            /* list radius is r_cut + skin */
  int32_t rebuild_every; /* rebuild after the drift of step k when (k+1) % rebuild_every == 0 */
  uint64_t seed;
} sn_md_params;

/* Caller-owned MD state; every pointer is a device buffer of R*N*3 floats,
 * except rowptr (R*N+1 int32) and col (edge_capacity int32). `step` counts the
 * steps taken so far and keys the noise: restoring (pos, vel, forces,
 * pos_at_build, rowptr, col, step) replays the same trajectory bit for bit.
 * rowptr_active (R*N+1 int32) and col_active (edge_capacity int32) are
 * optional, both NULL or both set: when set, the MD calls copy from the skin
 * list (rowptr, col), after every drift, the pairs closer than
 * r_cut (1 + 2^-10) by the list's own membership test, and evaluate energies
 * and forces on those. Listed pairs at or beyond r_cut contribute nothing,
 * so the results are the skin list's (up to the order of the force sums)
 * for less work; the active list is rebuilt from the state each step and
 * needs no restoring. Skins below r_cut 2^-10 skip the copy. */
typedef struct {
  float* pos;
  float* vel;
  float* forces;
  float* pos_at_build;
  int32_t* rowptr;
  int32_t* col;
  int64_t edge_capacity;
  uint64_t step;
  int32_t* rowptr_active;
  int32_t* col_active;
} sn_md_state;

/* Draws Maxwell-Boltzmann velocities (Philox counter (atom, 0, 1, 0)), builds
 * the list at r_cut + skin, evaluates forces and records pos_at_build.
 * energy[R] is optional (may be NULL). Periodic positions are wrapped into
 * [0, box) first. */
sn_status sn_md_init(const sn_model* model, const sn_system* sys, const int32_t* types,
                     const sn_md_params* params, sn_md_state* state, float* energy, void* ws,
                     size_t ws_bytes, hipStream_t stream);

/* Advances n_steps BAOAB steps for all replicas and adds n_steps to
 * state->step. Besides the scheduled rebuilds, the list is rebuilt on the
 * device after any step in which some atom moved more than skin/2 since the
 * last build. energy[R] (optional) receives the potential energy after the
 * last step. Periodic positions are wrapped into [0, box) after each drift.
 * An atom i whose position or velocity becomes NaN or infinite in a step sets
 * the device status to SN_ERR_NONFINITE with detail -(1 + i); the state is
 * then invalid (restore a checkpoint). */
sn_status sn_md_step(const sn_model* model, const sn_system* sys, const int32_t* types,
                     const sn_md_params* params, sn_md_state* state, int32_t n_steps,
                     float* energy, void* ws, size_t ws_bytes, hipStream_t stream);

/* Reads the device status word and its detail (synchronises the stream):
 * status_host gets an sn_status value; detail_host the needed edge count for
 * SN_ERR_CAPACITY; for SN_ERR_NONFINITE the replica r >= 0 whose energy is
 * not finite, or -(1 + i) for atom i whose position or velocity is not
 * finite; for SN_ERR_INVALID_ARG an atom whose type is out of range; for
 * SN_ERR_UNSUPPORTED the edge count of a list too long to evaluate.
 * n_rebuilds_host (may be
 * NULL) gets the number of neighbour-list builds done by the MD calls. */
sn_status sn_get_device_status(const void* ws, size_t ws_bytes, hipStream_t stream,
                               int32_t* status_host, int64_t* detail_host,
                               int64_t* n_rebuilds_host);

/* Work counters of the workspace (synchronises the stream): the number of
 * fused energy + force evaluations (sn_energy_forces, and those inside the
 * MD calls) enqueued on it since the last sn_reset_device_status, and the
 * sum of the edge counts rowptr[R*N] of the lists they ran on (the MD calls
 * evaluate the active list when the state has one). */
sn_status sn_get_device_counters(const void* ws, size_t ws_bytes, hipStream_t stream,
                                 int64_t* evaluations_host, int64_t* edges_evaluated_host);

/* Zeroes the status word and the counters (enqueued on the stream). */
sn_status sn_reset_device_status(void* ws, size_t ws_bytes, hipStream_t stream);

const char* sn_status_string(sn_status status);

/* Test hook: out[i][0..3] = Philox4x64-10(counter = counters[i][0..3],
 * key = (key0, key1)) for i < n, the generator behind the MD noise. */
sn_status sn_philox4x64_10(const uint64_t* counters, uint64_t key0, uint64_t key1, uint64_t* out,
                           int64_t n, hipStream_t stream);

/* Profiling hook: while enabled, the library records a pair of HIP events on
 * the launch stream around every launch of the fused CFConv kernels, so their
 * average device time can be read while other work runs. kernel: 0 = forward
 * CFConv, 1 = backward CFConv (forces). sn_profile_read synchronises on the
 * recorded events and returns the summed milliseconds and launch count since
 * the last read (it then starts a new tally). */
sn_status sn_profile_enable(int32_t on);
sn_status sn_profile_read(int32_t kernel, double* total_ms_host, int64_t* launches_host);

#ifdef __cplusplus
}
#endif
#endif /* SCHNET_MI355X_H */
