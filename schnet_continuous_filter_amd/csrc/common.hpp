// Internal declarations shared by the HIP translation units of the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "schnet_mi355x.h"

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

namespace sn {

constexpr int kThreads = 256;  // every kernel of the library runs 4 wave64 per block
constexpr int kMaxWorkers = 8192; // upper bound on CFConv workers (partition table size)
constexpr int kCellsPerAxisMax = 64;
constexpr int kOpenCellMinAtoms = 8192;   // open single systems this large use a cell list
constexpr int kScanChunk = 1024; // elements per block of the device scan
constexpr int kSortRowMax = 1024;

// Device status block at offset 0 of every workspace.
struct DevStatus {
  int32_t status;        // sn_status; first error wins
  int32_t overflow;      // 1 while the last neighbour build did not fit
  int64_t detail;
  int64_t n_rebuilds;    // neighbour builds done by the MD calls
  int64_t last_n_edges;  // edge count of the last neighbour build
  int64_t rebuild_req;   // MD: step+1 of the last step whose drift crossed skin/2
  int64_t evaluations;   // fused energy + force evaluations enqueued since the last reset
  int64_t edges_evaluated;   // the sum of their lists' edge counts
  int64_t pad[1];
};

// MLP operand precisions (the filter_dtype values of sn_model_desc): fp32;
// bfloat16 filter network; fp16 operands with per-output-channel power-of-two
// scales in every MLP; fp32 filter network evaluated on fp16 hi/lo pairs.
enum Prec { PREC_F32 = 0, PREC_BF16 = 1, PREC_F16S = 2, PREC_F16X2 = 3 };

// Round-to-nearest-even bfloat16 bits of a finite float (host side).
inline uint16_t bf16_rne_bits(float f) {
  uint32_t u;
  __builtin_memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// IEEE binary16 bits of a float, round to nearest even (host side).
inline uint16_t f16_rne_bits(float f) {
  const _Float16 h = (_Float16)f;
  uint16_t u;
  __builtin_memcpy(&u, &h, 2);
  return u;
}

// Per-output-channel scale of a weight matrix for fp16 operands: the power of
// two at or above the column's largest magnitude (1 for an all-zero column),
// so that W / s lies in [-1, 1] and the division is exact.
inline float pow2_scale(float absmax) {
  if (!(absmax > 0.f)) return 1.f;
  int e = 0;
  const float m = __builtin_frexpf(absmax, &e);   // absmax = m 2^e, m in [0.5, 1)
  (void)m;
  return __builtin_ldexpf(1.f, e);
}

__device__ inline void dev_fail(DevStatus* st, int code, int64_t detail) {
  if (atomicCAS(&st->status, 0, code) == 0) st->detail = detail;
}

// Offsets (bytes) of everything carved out of a workspace.
struct WsLayout {
  size_t status, wg_start, wg_start_b, wg_start_b0, wg_edge, wg_edge_b, wg_edge_b0, side_h, side_f;
  size_t scan_blocks, cell_count, cell_start, cell_atoms, atom_cell, cell_grid;
  size_t x, au, gbuf, tmp, gx, fblk, eps, total;
};
WsLayout ws_layout(int64_t n_atoms, int D, int T, int H);

// ------------------------------------------------------------------ launchers
// Neighbour list (nbr.hip). Returns hipSuccess or the first launch error.
struct NbrGeom {
  int n_rep, n_per, periodic;
  float box;
  double L, half, r2;   // IEEE double values used by the exact predicate
  int cells_per_axis;   // 0 = all-pairs mode; -1 = cell list over the bounding box (open system)
  float inv_cell;
};
hipError_t launch_build_neighbors(const NbrGeom& g, const float* pos, int32_t* rowptr,
                                  int32_t* col, int64_t edge_capacity, char* ws,
                                  const WsLayout& L, const int64_t* gate, int64_t gate_val,
                                  hipStream_t s);

// Rows of (rowptr, col) restricted to the pairs inside sqrt(r2) by the same
// membership test, same order, into (out_rowptr [n+1], out_col) (nbr.hip).
hipError_t launch_active_list(const NbrGeom& g, const float* pos, const int32_t* rowptr,
                              const int32_t* col, double r2, int32_t* out_rowptr,
                              int32_t* out_col, char* ws, const WsLayout& L, hipStream_t s);

// Scan (nbr.hip): in-place exclusive scan of a[0..n) into a[0..n], a[n] = total.
hipError_t launch_exclusive_scan(int32_t* a, int64_t n, int32_t* blocks, DevStatus* st,
                                 int64_t capacity, const int64_t* gate, int64_t gate_val,
                                 hipStream_t s);

// CFConv and atom-wise layers (cfconv.hip, atomwise.hip).
struct CfParams {
  const int32_t* rowptr;
  const int32_t* col;
  const float* pos;
  const int32_t* wg_start;  // per worker: first receiver (launch_setup)
  const int32_t* wg_edge;   // per worker: first edge (a multiple of 16)
  // receivers cut by worker boundaries: the part a worker holds of its last,
  // unfinished receiver (side_h [workers][D] features, side_f [workers][3]
  // force rows); the worker holding the receiver's last edge writes its own
  // part to the output, and the kernels that next read that output add the
  // other parts (cut_workers names the workers)
  float* side_h;
  float* side_f;
  int n_atoms;
  int periodic;
  float box, half_box;
  float rbf_min, rbf_step, rbf_coef2, rbf_inv_s2; // coef2 = -log2(e)/(2 sigma^2), inv_s2 = 1/sigma^2
  // neighbouring Gaussians: g_{k+1} / g_k = 2^(qa z_k + qb) with z_k = d - mu_k,
  // and that ratio shrinks by the factor r from one k to the next
  float rbf_qa, rbf_qb, rbf_r;
  float r_cut, pi_over_rc, half_over_rc;   // half_over_rc = 1 / (2 r_cut)
  int KC;             // basis chunks the first filter product runs over (cf_chunks)
  const void* img;    // this block's filter weights and biases as laid out in LDS (cf_fill_image)
  const float* x;     // x^(t) [N][D]
  float* h;           // forward output [N][D]
  const float* gh;    // backward: dE/dh^(t) [N][D]
  float* q_out;       // backward: sum_j dE/dh_j w_ij [N][D], or null for the first block
  float* forces;      // backward: this block's dE/dr [N][3]
};

// prec: the model's filter_dtype (Prec).
int cf_kp(int Dr, int prec);               // basis length the LDS images are padded to
int cf_chunks(int Dr, int prec);           // basis chunks (8 fp32 / 32 16-bit basis functions each)
// waves (workers) per work-group of a kernel: kind 0 the forward, 1 the
// backward, 2 the backward of the first block (no source sums)
int cf_workers(int D, int KP, int prec, int kind);
hipError_t cf_prepare(int D, int KP, int prec);  // raises the dynamic LDS limit of the kernels
// Filter-weight image of one interaction block as the CFConv kernels hold it
// in LDS: cf_image_bytes bytes, filled on the host.
size_t cf_image_bytes(int D, int KP, int prec);
// rbf_step and r_cut bound the basis functions and their derivatives, from
// which PREC_F16X2 sets the power-of-two scales of its product inputs.
void cf_fill_image(int D, int KP, int prec, int Dr, const float* Wf1, const float* cf1,
                   const float* Wf2, const float* cf2, float rbf_step, float r_cut,
                   unsigned char* out);
// MD bookkeeping that joins the set-up launch: when *gate == gate_val (or
// gate is null), the positions of a list build are kept (pos_at_build =
// pos) and the build is counted (DevStatus::n_rebuilds).
struct BuildMark {
  const float* pos;
  float* pos_at_build;
  const int64_t* gate;
  int64_t gate_val;
};
// The CFConv kernels' worker partitions of the receiver CSR (G1 workers of
// the forward, G2 of the backward, G3 of the first block's backward; skipped
// when rowptr is null), the initial features x = Emb[types] and, with mark,
// the build mark, in one launch (x null: the features are left as they are).
hipError_t launch_setup(const int32_t* rowptr, int n_atoms, int G1, int32_t* wg_start1,
                        int32_t* wg_edge1, int G2, int32_t* wg_start2, int32_t* wg_edge2,
                        int G3, int32_t* wg_start3, int32_t* wg_edge3, const int32_t* types,
                        const float* emb, int D, int n_types, float* x, const BuildMark* mark,
                        DevStatus* st, hipStream_t s);
hipError_t launch_cf_forward(int D, int KP, int prec, const CfParams& p, int G, hipStream_t s);
hipError_t launch_cf_backward(int D, int KP, int prec, const CfParams& p, int G, hipStream_t s);

enum AtomMode { ATOM_UPDATE_FWD = 0, ATOM_UPDATE_BWD = 1, ATOM_READOUT = 2 };
struct AtomArgs {
  int mode;
  int M;              // atoms
  const float* A;     // [M][D]: h (update fwd), dE/dx' (update bwd), x^(T) (readout)
  const float* A2;    // update bwd: added to A when not null (the CFConv source sum)
  float* Asum;        // update bwd: A + A2 is stored here when not null
  const float* R;     // residual x [M][D] (update fwd)
  const float* S;     // pre-activation a [M][N1] (update bwd)
  float* Aout;        // pre-activation a [M][N1] (update fwd)
  float* Y;           // [M][D]: x', dE/dh, or dE/dx^(T)
  float b2s;          // readout output bias
  float* eps;         // per-atom energies [M] (readout)
  const void* img;    // the network's weight image (atom_fill_image)
  // receivers of the CFConv launch (cut_G workers over the list cut_rowptr)
  // that wrote A (update fwd) or A2 (update bwd) whose parts cut_side
  // [workers][D] holds; null: none
  const int32_t* cut_rowptr;
  int cut_G;
  const float* cut_side;
};
// Weight image of one atom-wise network for `mode`: W1 [D][N1], b1 [N1],
// W2 [N1][D] (readout: wo2 [N1]), b2 [D]; built on the host.
// prec: the model's filter_dtype (Prec). The atom-wise layers take fp16
// operands for PREC_F16S, fp16 pairs for PREC_F16X2 and PREC_BF16 (behind a
// bfloat16 filter they stay fp32-grade), fp32 operands for PREC_F32; the
// fused and the unfused pipelines run the same atom-wise kernels.
size_t atom_image_bytes(int D, int N1, int prec);
void atom_fill_image(int mode, int D, int N1, int prec, const float* W1, const float* b1,
                     const float* W2, const float* b2, unsigned char* out);
hipError_t atom_prepare(int D, int H, int prec);   // raises the dynamic LDS limit of the kernels
hipError_t launch_atom(const AtomArgs& g, int D, int N1, int prec, int n_cu, hipStream_t s);
// Per-replica energies (double sums of eps) and F = -(sum over the T blocks
// of fb), in one launch; with vel, also vel += half_kick F. With side_f,
// block t's rows of receivers cut by the workers of its CFConv launch (G0
// for block 0, G for the others, over the list rowptr) gain their parts
// side_f[t * side_stride + 3 w].
hipError_t launch_finish(const float* eps, int n_rep, int n_per, float* energy, const float* fb,
                         int T, int64_t n_atoms, float* forces, float* vel, float half_kick,
                         const int32_t* rowptr, int G0, int G, const float* side_f,
                         int64_t side_stride, DevStatus* st, hipStream_t s);

// Unfused edge pipeline (unfused.hip): one kernel per step, edge tensors in
// the workspace, atomic or segmented aggregation.
enum UfPhase { UF_EDGES = 0, UF_FORWARD = 1, UF_BACKWARD = 2 };
struct UfImages { size_t g1, g2, g3, g4, total; };  // byte offsets of the four product images
struct UfArgs {
  int phase, atomic;
  int D, KP, Dr, bf16, n_cu, n_atoms, periodic;
  int64_t cap;                 // edge capacity (rows of every edge tensor)
  float box, rbf_min, rbf_step, r_cut;
  const int32_t* rowptr;
  const int32_t* col;
  const float* pos;
  DevStatus* st;
  // per call: indices, geometry, basis, dE/dr
  int32_t* dst;                // [cap] receiver of each edge
  int32_t* rev;                // [cap] reverse edge (segmented mode)
  f32x4* geo;                  // [cap] (u, d)
  float* B;                    // [cap][KP] basis
  float* C;                    // [cap] envelope
  float* mask;                 // [cap] 1 inside the cutoff
  float* gd;                   // [cap] dE/dd
  float* gB;                   // [cap][KP] dE/dB
  float* dEdr;                 // [N][3] accumulated over blocks
  // per block
  const void* img;             // uf_fill_images of this block
  const float* cf1;
  const float* cf2;
  const float* x;              // x^(t) [N][D]
  float* h;                    // forward output [N][D]
  const float* gh;             // backward input dE/dh [N][D]
  float* q;                    // backward sender sums [N][D], or null
  float* A;                    // [cap][D] filter pre-activation (kept for the backward)
  float* W;                    // [cap][D] masked filter (kept)
  float* Xs;                   // [cap][D] gathered sender rows (kept)
  float* buf0;                 // [cap][D] scratch
  float* buf1;
  float* buf2;
};
UfImages uf_images(int D, int KP, int bf16);
void uf_fill_images(int D, int KP, int bf16, int Dr, const float* Wf1, const float* Wf2,
                    unsigned char* out);
hipError_t uf_prepare(int D, int KP, int bf16);
hipError_t launch_unfused(const UfArgs& a, hipStream_t s);

// MD (md.hip).
struct MdCoef {
  float half_kick;   // dt/2 * kappa / m
  float half_dt;     // dt/2
  float c1, c2;      // O-step coefficients
  float sigma_v;     // Maxwell-Boltzmann width
  float half_skin2;  // (skin/2)^2
  uint64_t seed;
  int periodic;
  float box;
};
hipError_t launch_md_init_vel(const MdCoef& c, int64_t n, float* vel, hipStream_t s);
hipError_t launch_md_wrap(const MdCoef& c, int64_t n, float* pos, hipStream_t s);
hipError_t launch_md_baoa(const MdCoef& c, int64_t n, uint64_t step, float* pos, float* vel,
                          const float* forces, const float* pos_at_build, DevStatus* st,
                          hipStream_t s);
hipError_t launch_philox(const uint64_t* ctr, uint64_t k0, uint64_t k1, uint64_t* out, int64_t n,
                         hipStream_t s);

} // namespace sn
