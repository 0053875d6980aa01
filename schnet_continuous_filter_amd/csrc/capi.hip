// C ABI: argument validation, workspace carving and launch orchestration.
// The calls and their contracts are documented in include/schnet_mi355x.h.
#include <cmath>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "common.hpp"

using namespace sn;

// Device memory of sn_energy_forces_noalloc (see scratch_for_current_device).
static __device__ __align__(256) unsigned char scratch[SN_SCRATCH_BYTES];

__global__ void k_status_clear(sn::DevStatus* st) {
  int64_t* w = reinterpret_cast<int64_t*>(st);
  constexpr int n = (int)(sizeof(sn::DevStatus) / sizeof(int64_t));
  if ((int)threadIdx.x < n) w[threadIdx.x] = 0;
}

__global__ void k_status_copy(const sn::DevStatus* st, int64_t* out) {
  if (threadIdx.x == 0) {
    out[0] = st->status;
    out[1] = st->detail;
  }
}

struct sn_model {
  sn_model_desc desc;
  int KP = 0;
  int n_cu = 0;
  size_t n_w = 0;
  float* w = nullptr;          // device copy of the flat fp32 weights
  unsigned char* cfimg = nullptr;  // per block: the CFConv weight image (cf_fill_image)
  size_t img_bytes = 0;
  unsigned char* atimg = nullptr;  // per block: update-forward then update-backward image; readout
  size_t at_upd = 0, at_ro = 0;     // image sizes (bytes)
  unsigned char* ufimg = nullptr;  // per block: the unfused pipeline's product images
  size_t uf_bytes = 0;
  float co2 = 0.f;             // readout output bias (host copy)
  size_t off_emb = 0, off_o1 = 0, off_co1 = 0, off_o2 = 0;
  std::vector<size_t> off_blk; // start of each interaction block
};

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t b) { return (b + kAlign - 1) / kAlign * kAlign; }

bool desc_ok(const sn_model_desc* d) {
  if (!d) return false;
  return d->n_types >= 1 && (d->D == 64 || d->D == 128) && d->Dr >= 2 && d->Dr <= 64 && d->T >= 1 &&
         d->T <= 8 && (d->H == 32 || d->H == 64) && d->H <= d->D && std::isfinite(d->rbf_min) &&
         std::isfinite(d->rbf_max) && d->rbf_min >= 0.f && d->rbf_max > d->rbf_min &&
         std::isfinite(d->r_cut) && d->r_cut > 0.f &&
         (d->filter_dtype == SN_FILTER_F32 || d->filter_dtype == SN_FILTER_BF16 ||
          d->filter_dtype == SN_W16A16 || d->filter_dtype == SN_FILTER_F16X2);
}

size_t block_floats(const sn_model_desc* d) {
  const size_t D = d->D, Dr = d->Dr;
  return Dr * D + D + 3 * (D * D + D);
}

bool sys_ok(const sn_system* s) {
  if (!s) return false;
  if (s->n_replicas < 1 || s->atoms_per_replica < 1) return false;
  // the kernels address per-atom feature rows with 32-bit byte offsets (N * 128 * 4 < 2^31)
  if ((int64_t)s->n_replicas * s->atoms_per_replica > ((int64_t)1 << 22)) return false;
  if (s->periodic && !(std::isfinite(s->box) && s->box > 0.f)) return false;
  return true;
}

int64_t n_atoms(const sn_system* s) { return (int64_t)s->n_replicas * s->atoms_per_replica; }

sn_status hip_fail(hipError_t e) { return e == hipSuccess ? SN_OK : SN_ERR_HIP; }

// ---------------------------------------------------------------- profiling hook
struct ProfRec { int kernel; hipEvent_t a, b; };
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRec> g_prof_recs;
std::vector<hipEvent_t> g_prof_pool;

hipEvent_t prof_event() {
  if (!g_prof_pool.empty()) {
    hipEvent_t e = g_prof_pool.back();
    g_prof_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

struct ProfScope {
  int kernel;
  hipStream_t s;
  hipEvent_t a = nullptr, b = nullptr;
  // kernel < 0: never recorded (the allocation-free entry point)
  ProfScope(int k, hipStream_t st) : kernel(k), s(st) {
    if (k < 0) return;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (!g_prof_on) return;
    a = prof_event();
    b = prof_event();
    if (a && b) (void)hipEventRecord(a, s);
  }
  ~ProfScope() {
    if (!(a && b)) return;
    (void)hipEventRecord(b, s);
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_recs.push_back({kernel, a, b});
  }
};

// ---------------------------------------------------------------- E+F orchestration
// Work-groups for a CFConv kernel: one per CU (its LDS plan allows one
// resident group), fewer only when there are not enough receivers to give
// every worker (wave) one.
int cf_grid(const sn_model* m, int64_t n, int workers) {
  int64_t g = (n + workers - 1) / workers;
  if (g > m->n_cu) g = m->n_cu;
  if (g * workers > kMaxWorkers) g = kMaxWorkers / workers;
  return (int)(g < 1 ? 1 : g);
}

// Edge tensors of the unfused pipeline, carved after the common workspace.
struct UfLayout {
  size_t dst, rev, geo, C, mask, gd, B, gB, keep, buf, total;
};
UfLayout uf_layout(size_t base, int64_t cap, int D, int KP, int T) {
  UfLayout U{};
  size_t off = base;
  auto take = [&](size_t bytes) { size_t o = off; off += align_up(bytes); return o; };
  const size_t c = (size_t)cap;
  U.dst = take(c * 4);
  U.rev = take(c * 4);
  U.geo = take(c * 16);
  U.C = take(c * 4);
  U.mask = take(c * 4);
  U.gd = take(c * 4);
  U.B = take(c * KP * 4);
  U.gB = take(c * KP * 4);
  U.keep = take((size_t)3 * T * c * D * 4);   // per block: A, W, X_src
  U.buf = take((size_t)3 * c * D * 4);
  U.total = off;
  return U;
}

struct UfMode {
  int64_t cap;
  int atomic;
};

sn_status energy_forces_impl(const sn_model* m, const sn_system* sys, const float* pos,
                             const int32_t* types, const int32_t* rowptr, const int32_t* col,
                             float* energy, float* forces, char* ws, hipStream_t s,
                             const UfMode* uf = nullptr, float* vel_kick = nullptr,
                             float half_kick = 0.f, const BuildMark* mark = nullptr,
                             bool profile = true, bool x0_ready = false) {
  const sn_model_desc& d = m->desc;
  const int64_t n = n_atoms(sys);
  const int D = d.D, T = d.T, H = d.H;
  const WsLayout L = ws_layout(n, D, T, H);
  DevStatus* st = reinterpret_cast<DevStatus*>(ws + L.status);
  int32_t* wg_start = reinterpret_cast<int32_t*>(ws + L.wg_start);
  int32_t* wg_start_b = reinterpret_cast<int32_t*>(ws + L.wg_start_b);
  int32_t* wg_edge = reinterpret_cast<int32_t*>(ws + L.wg_edge);
  int32_t* wg_edge_b = reinterpret_cast<int32_t*>(ws + L.wg_edge_b);
  int32_t* wg_start_b0 = reinterpret_cast<int32_t*>(ws + L.wg_start_b0);
  int32_t* wg_edge_b0 = reinterpret_cast<int32_t*>(ws + L.wg_edge_b0);
  float* x = reinterpret_cast<float*>(ws + L.x);
  float* au = reinterpret_cast<float*>(ws + L.au);
  float* gbuf = reinterpret_cast<float*>(ws + L.gbuf);
  float* tmp = reinterpret_cast<float*>(ws + L.tmp);
  float* gx = reinterpret_cast<float*>(ws + L.gx);
  float* eps = reinterpret_cast<float*>(ws + L.eps);
  float* fblk = reinterpret_cast<float*>(ws + L.fblk);
  const size_t ND = (size_t)n * D;
  const int prec = d.filter_dtype;
  const int bf16 = prec == PREC_BF16;
  // workers of the forward, the backward and the first block's backward
  const int wf = cf_workers(D, m->KP, prec, 0), wb = cf_workers(D, m->KP, prec, 1),
            wb0 = cf_workers(D, m->KP, prec, 2);
  const int Gf = cf_grid(m, n, wf), Gb = cf_grid(m, n, wb), Gb0 = cf_grid(m, n, wb0);
  hipError_t e;

  // x0_ready: the workspace already holds x0 = Emb[types] for these types
  if ((e = launch_setup(uf ? nullptr : rowptr, (int)n, Gf * wf, wg_start, wg_edge, Gb * wb,
                        wg_start_b, wg_edge_b, Gb0 * wb0, wg_start_b0, wg_edge_b0, types,
                        m->w + m->off_emb, D, d.n_types, x0_ready ? nullptr : x, mark, st,
                        s)) != hipSuccess)
    return hip_fail(e);

  CfParams p{};
  p.rowptr = rowptr;
  p.col = col;
  p.pos = pos;
  p.wg_start = wg_start;
  p.wg_edge = wg_edge;
  p.side_h = reinterpret_cast<float*>(ws + L.side_h);
  float* side_f = reinterpret_cast<float*>(ws + L.side_f);   // one [workers][3] array per block
  constexpr int64_t kSideF = (int64_t)kMaxWorkers * 3;
  p.n_atoms = (int)n;
  p.periodic = sys->periodic;
  p.box = sys->box;
  p.half_box = 0.5f * sys->box;
  const float step = (d.rbf_max - d.rbf_min) / (float)(d.Dr - 1);
  p.rbf_min = d.rbf_min;
  p.rbf_step = step;
  p.rbf_coef2 = (float)(-0.5 / ((double)step * step) * 1.4426950408889634);
  p.rbf_inv_s2 = 1.f / (step * step);
  {
    // sigma = step: g_{k+1} / g_k = exp((z_k step - step^2 / 2) / sigma^2)
    const double st = step, is2 = 1.0 / ((double)step * step), l2e = 1.4426950408889634;
    p.rbf_qa = (float)(l2e * st * is2);
    p.rbf_qb = (float)(-0.5 * l2e * st * st * is2);
    p.rbf_r = (float)std::exp(-st * st * is2);
  }
  p.r_cut = d.r_cut;
  p.pi_over_rc = (float)(M_PI / (double)d.r_cut);
  p.half_over_rc = (float)(0.5 / (double)d.r_cut);
  p.KC = cf_chunks(d.Dr, prec);

  auto block_img = [&](int t) -> const void* { return m->cfimg + (size_t)t * m->img_bytes; };
  auto Wu = [&](int t, int k) {  // k: 0 Wu1, 1 cu1, 2 Wu2, 3 cu2
    const float* b = m->w + m->off_blk[t] + (size_t)d.Dr * D + D + (size_t)D * D + D;
    const size_t DD = (size_t)D * D;
    switch (k) {
      case 0: return b;
      case 1: return b + DD;
      case 2: return b + DD + D;
      default: return b + 2 * DD + D;
    }
  };

  auto atom_img = [&](int t, int bwd) -> const void* {
    return m->atimg + (size_t)t * 2 * m->at_upd + (bwd ? m->at_upd : 0);
  };
  const void* ro_img = m->atimg + (size_t)T * 2 * m->at_upd;

  UfArgs ua{};
  float* uf_keep = nullptr;
  if (uf) {
    const UfLayout U = uf_layout(L.total, uf->cap, D, m->KP, T);
    uf_keep = reinterpret_cast<float*>(ws + U.keep);
    ua.atomic = uf->atomic;
    ua.D = D;
    ua.KP = m->KP;
    ua.Dr = d.Dr;
    ua.bf16 = bf16;
    ua.n_cu = m->n_cu;
    ua.n_atoms = (int)n;
    ua.periodic = sys->periodic;
    ua.cap = uf->cap;
    ua.box = sys->box;
    ua.rbf_min = d.rbf_min;
    ua.rbf_step = step;
    ua.r_cut = d.r_cut;
    ua.rowptr = rowptr;
    ua.col = col;
    ua.pos = pos;
    ua.st = st;
    ua.dst = reinterpret_cast<int32_t*>(ws + U.dst);
    ua.rev = reinterpret_cast<int32_t*>(ws + U.rev);
    ua.geo = reinterpret_cast<f32x4*>(ws + U.geo);
    ua.B = reinterpret_cast<float*>(ws + U.B);
    ua.C = reinterpret_cast<float*>(ws + U.C);
    ua.mask = reinterpret_cast<float*>(ws + U.mask);
    ua.gd = reinterpret_cast<float*>(ws + U.gd);
    ua.gB = reinterpret_cast<float*>(ws + U.gB);
    ua.dEdr = fblk;
    const size_t ED = (size_t)uf->cap * D;
    ua.buf0 = reinterpret_cast<float*>(ws + U.buf);
    ua.buf1 = ua.buf0 + ED;
    ua.buf2 = ua.buf1 + ED;
    ua.phase = UF_EDGES;
    if ((e = launch_unfused(ua, s)) != hipSuccess) return hip_fail(e);
  }
  auto uf_block = [&](int t, int phase) {
    const size_t ED = (size_t)uf->cap * D;
    ua.phase = phase;
    ua.img = m->ufimg + (size_t)t * m->uf_bytes;
    const float* Wf1 = m->w + m->off_blk[t];
    ua.cf1 = Wf1 + (size_t)d.Dr * D;
    ua.cf2 = ua.cf1 + D + (size_t)D * D;
    ua.A = uf_keep + (size_t)3 * t * ED;
    ua.W = ua.A + ED;
    ua.Xs = ua.W + ED;
    ua.x = x + t * ND;
    return launch_unfused(ua, s);
  };

  // forward
  for (int t = 0; t < T; ++t) {
    p.img = block_img(t);
    p.wg_start = wg_start;
    p.wg_edge = wg_edge;
    p.x = x + t * ND;
    p.h = gbuf;
    if (uf) {
      ua.h = gbuf;
      if ((e = uf_block(t, UF_FORWARD)) != hipSuccess) return hip_fail(e);
    } else {
      ProfScope ps(profile ? 0 : -1, s);
      if ((e = launch_cf_forward(D, m->KP, prec, p, Gf, s)) != hipSuccess) return hip_fail(e);
    }
    // h of receivers cut by the forward's worker boundaries is completed as it is read
    AtomArgs u{ATOM_UPDATE_FWD, (int)n, gbuf, nullptr, nullptr, x + t * ND, nullptr, au + t * ND,
               x + (t + 1) * ND, 0.f, nullptr, atom_img(t, 0)};
    if (!uf) {
      u.cut_rowptr = rowptr;
      u.cut_G = Gf * wf;
      u.cut_side = p.side_h;
    }
    if ((e = launch_atom(u, D, D, prec, m->n_cu, s)) != hipSuccess) return hip_fail(e);
  }
  // readout and its gradient
  AtomArgs r{ATOM_READOUT, (int)n, x + T * ND, nullptr, nullptr, nullptr, nullptr, nullptr, gx,
             m->co2, eps, ro_img};
  if ((e = launch_atom(r, D, H, prec, m->n_cu, s)) != hipSuccess) return hip_fail(e);
  // backward: gx holds dE/dx^(t+1) without the newest source sum q, which the
  // update-backward kernel adds (and stores back while an older block needs it)
  for (int t = T - 1; t >= 0; --t) {
    const bool has_q = t < T - 1;
    AtomArgs b{ATOM_UPDATE_BWD, (int)n, gx, has_q ? tmp : nullptr, (has_q && t > 0) ? gx : nullptr,
               nullptr, au + t * ND, nullptr, gbuf, 0.f, nullptr, atom_img(t, 1)};
    if (!uf && has_q) {   // q of the previous backward launch, completed as it is read
      b.cut_rowptr = rowptr;
      b.cut_G = Gb * wb;
      b.cut_side = p.side_h;
    }
    if ((e = launch_atom(b, D, D, prec, m->n_cu, s)) != hipSuccess) return hip_fail(e);
    // the first block (no source sums) runs its own kernel and partition
    p.img = block_img(t);
    p.wg_start = t > 0 ? wg_start_b : wg_start_b0;
    p.wg_edge = t > 0 ? wg_edge_b : wg_edge_b0;
    p.x = x + t * ND;
    p.gh = gbuf;
    p.q_out = t > 0 ? tmp : nullptr;
    p.forces = fblk + (size_t)t * n * 3;
    p.side_f = side_f + t * kSideF;
    if (uf) {
      ua.gh = gbuf;
      ua.q = t > 0 ? tmp : nullptr;
      if ((e = uf_block(t, UF_BACKWARD)) != hipSuccess) return hip_fail(e);
    } else {
      ProfScope ps(profile ? 1 : -1, s);
      if ((e = launch_cf_backward(D, m->KP, prec, p, t > 0 ? Gb : Gb0, s)) != hipSuccess)
        return hip_fail(e);
    }
  }
  // replica energies, and the forces (the unfused pipeline accumulates dE/dr
  // of every block into one array), each block's rows of cut receivers
  // completed from its side parts
  if ((e = launch_finish(eps, sys->n_replicas, sys->atoms_per_replica, energy, fblk, uf ? 1 : T, n,
                         forces, vel_kick, half_kick, rowptr, Gb0 * wb0, Gb * wb,
                         uf ? nullptr : side_f, kSideF, st, s)) != hipSuccess)
    return hip_fail(e);
  return SN_OK;
}

// ---------------------------------------------------------------- allocation-free workspace
// The workspace of sn_energy_forces_noalloc: a static device array, one copy
// per GPU (the loader places it when the library's code object is loaded on
// that GPU; it is held until the process ends). Host code never uses the
// array's name as an address: the device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
constexpr size_t kScratchBytes = SN_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

sn_status scratch_for_current_device(char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SN_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return SN_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return SN_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = static_cast<char*>(g_scratch_ptr[dev]);
  return SN_OK;
}

sn_status check_ws(const void* ws, size_t ws_bytes, size_t need) {
  if (!ws) return SN_ERR_INVALID_ARG;
  if (((uintptr_t)ws) % kAlign != 0) return SN_ERR_INVALID_ARG;
  return ws_bytes >= need ? SN_OK : SN_ERR_WORKSPACE;
}

bool nbr_geom(const sn_system* sys, float r_list, NbrGeom& g) {
  if (!(std::isfinite(r_list) && r_list > 0.f)) return false;
  g.n_rep = sys->n_replicas;
  g.n_per = sys->atoms_per_replica;
  g.periodic = sys->periodic != 0;
  g.box = sys->box;
  g.L = g.periodic ? (double)sys->box : 0.0;
  g.half = g.L / 2.0;
  g.r2 = (double)r_list * (double)r_list;
  g.cells_per_axis = 0;
  g.inv_cell = 0.f;
  if (g.periodic) {
    if (!((double)sys->box >= 2.0 * (double)r_list)) return false;
    int nc = (int)std::floor((double)sys->box / ((double)r_list * (1.0 + 1e-5)));
    if (nc > kCellsPerAxisMax) nc = kCellsPerAxisMax;
    // cells hold every replica's atoms (the pair test keeps replicas apart),
    // so several replicas take them only when each is large
    if (nc >= 3 && (sys->n_replicas == 1 || sys->atoms_per_replica >= kOpenCellMinAtoms)) {
      g.cells_per_axis = nc;
      g.inv_cell = (float)((double)nc / (double)sys->box);
    }
  } else if (sys->atoms_per_replica >= kOpenCellMinAtoms) {
    g.cells_per_axis = -1;   // grid over the bounding box of all replicas, set on the device
  }
  return true;
}

struct MdSetup {
  MdCoef c;
  float r_list;
};

bool md_setup(const sn_model* m, const sn_system* sys, const sn_md_params* prm, MdSetup& out) {
  if (!prm) return false;
  if (!(prm->dt_fs > 0.f && std::isfinite(prm->dt_fs)) || !(prm->temperature_K >= 0.f) ||
      !(prm->gamma_per_ps >= 0.f) || !(prm->mass_amu > 0.f) || !(prm->skin >= 0.f) ||
      prm->rebuild_every < 1)
    return false;
  const double kappa = 4.184e-4, kB = 0.0019872043;
  const double dt = prm->dt_fs, m_ = prm->mass_amu;
  const double c1 = std::exp(-(double)prm->gamma_per_ps * 1e-3 * dt);
  out.c.half_kick = (float)(0.5 * dt * kappa / m_);
  out.c.half_dt = (float)(0.5 * dt);
  out.c.c1 = (float)c1;
  out.c.c2 = (float)std::sqrt((1.0 - c1 * c1) * kB * prm->temperature_K * kappa / m_);
  out.c.sigma_v = (float)std::sqrt(kB * prm->temperature_K * kappa / m_);
  out.c.half_skin2 = (float)(0.25 * (double)prm->skin * prm->skin);
  out.c.seed = prm->seed;
  out.c.periodic = sys->periodic != 0;
  out.c.box = sys->box;
  out.r_list = m->desc.r_cut + prm->skin;
  return true;
}

bool state_ok(const sn_md_state* st) {
  return st && st->pos && st->vel && st->forces && st->pos_at_build && st->rowptr && st->col &&
         st->edge_capacity >= 0 && st->edge_capacity <= INT32_MAX &&
         (st->rowptr_active == nullptr) == (st->col_active == nullptr);
}

// The list the MD calls evaluate: the active list (pairs inside r_cut plus a
// margin of 2^-10 r_cut, far above the rounding of the kernels' distances),
// copied from the skin list after the drift when the state provides its
// buffers and the skin is wider than the margin; the skin list otherwise.
hipError_t md_eval_list(const sn_model* m, const sn_md_params* prm, const NbrGeom& g,
                        const sn_md_state* state, char* w, const WsLayout& L, hipStream_t s,
                        const int32_t*& rp, const int32_t*& cl) {
  rp = state->rowptr;
  cl = state->col;
  const double margin = (double)m->desc.r_cut / 1024.0;
  if (!state->rowptr_active || !((double)prm->skin > margin)) return hipSuccess;
  const double rk = (double)(float)((double)m->desc.r_cut + margin);
  rp = state->rowptr_active;
  cl = state->col_active;
  return launch_active_list(g, state->pos, state->rowptr, state->col, rk * rk,
                            state->rowptr_active, state->col_active, w, L, s);
}

} // namespace

namespace sn {
WsLayout ws_layout(int64_t n, int D, int T, int H) {
  (void)H;
  WsLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align_up(bytes); return o; };
  const int64_t ncell = (int64_t)kCellsPerAxisMax * kCellsPerAxisMax * kCellsPerAxisMax;
  const int64_t scan_n = (n > ncell ? n : ncell) + 1;
  L.status = take(sizeof(DevStatus));
  L.wg_start = take((size_t)(kMaxWorkers + 1) * 4);
  L.wg_start_b = take((size_t)(kMaxWorkers + 1) * 4);
  L.wg_edge = take((size_t)(kMaxWorkers + 1) * 4);
  L.wg_edge_b = take((size_t)(kMaxWorkers + 1) * 4);
  L.wg_start_b0 = take((size_t)(kMaxWorkers + 1) * 4);
  L.wg_edge_b0 = take((size_t)(kMaxWorkers + 1) * 4);
  L.side_h = take((size_t)kMaxWorkers * (size_t)D * 4);
  L.side_f = take((size_t)T * kMaxWorkers * 3 * 4);
  L.scan_blocks = take((size_t)(scan_n / kScanChunk + 2) * 8);
  L.cell_count = take((size_t)(ncell + 1) * 4);
  L.cell_start = take((size_t)ncell * 4);
  L.cell_atoms = take((size_t)n * 4);
  L.atom_cell = take((size_t)n * 4);
  L.cell_grid = take(64);
  const size_t ND = (size_t)n * (size_t)D * 4;
  L.x = take((size_t)(T + 1) * ND);
  L.au = take((size_t)T * ND);
  L.gbuf = take(ND);
  L.tmp = take(ND);
  L.gx = take(ND);
  L.fblk = take((size_t)T * n * 3 * 4);          // per-block dE/dr
  L.eps = take((size_t)n * 4 + (size_t)n * 4);   // per-atom energies, then per-replica scratch
  L.total = off;
  return L;
}
} // namespace sn

extern "C" {

const char* sn_status_string(sn_status s) {
  switch (s) {
    case SN_OK: return "ok";
    case SN_ERR_INVALID_ARG: return "invalid argument";
    case SN_ERR_CAPACITY: return "neighbour list exceeds edge capacity";
    case SN_ERR_NONFINITE: return "non-finite energy, position or velocity";
    case SN_ERR_UNSUPPORTED: return "unsupported shape";
    case SN_ERR_HIP: return "HIP runtime error";
    case SN_ERR_WORKSPACE: return "workspace too small";
  }
  return "unknown status";
}

size_t sn_model_weight_count(const sn_model_desc* d) {
  if (!desc_ok(d)) return 0;
  const size_t D = d->D, H = d->H;
  return (size_t)d->n_types * D + (size_t)d->T * block_floats(d) + D * H + H + H + 1;
}

sn_status sn_model_create(const sn_model_desc* d, const float* weights_host, size_t n_floats,
                          sn_model** out) {
  if (!d || !weights_host || !out) return SN_ERR_INVALID_ARG;
  *out = nullptr;
  if (!desc_ok(d)) {
    // distinguish malformed values from shapes this build does not cover
    if (d->n_types < 1 || d->D < 1 || d->Dr < 2 || d->T < 1 || d->H < 1 ||
        !(d->rbf_max > d->rbf_min) || !(d->r_cut > 0.f))
      return SN_ERR_INVALID_ARG;
    return SN_ERR_UNSUPPORTED;
  }
  const size_t nw = sn_model_weight_count(d);
  if (n_floats != nw) return SN_ERR_INVALID_ARG;
  for (size_t i = 0; i < nw; ++i)
    if (!std::isfinite(weights_host[i])) return SN_ERR_INVALID_ARG;

  sn_model* m = new (std::nothrow) sn_model();
  if (!m) return SN_ERR_HIP;
  m->desc = *d;
  m->n_w = nw;
  m->KP = cf_kp(d->Dr, d->filter_dtype);
  const size_t D = d->D, H = d->H;
  m->off_emb = 0;
  size_t off = (size_t)d->n_types * D;
  for (int t = 0; t < d->T; ++t) {
    m->off_blk.push_back(off);
    off += block_floats(d);
  }
  m->off_o1 = off;
  m->off_co1 = off + D * H;
  m->off_o2 = m->off_co1 + H;
  m->co2 = weights_host[m->off_o2 + H];

  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&m->n_cu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) e = cf_prepare(d->D, m->KP, d->filter_dtype);
  if (e == hipSuccess) e = hipMalloc(&m->w, nw * sizeof(float));
  if (e == hipSuccess) e = hipMemcpy(m->w, weights_host, nw * sizeof(float), hipMemcpyHostToDevice);
  if (e == hipSuccess) {
    // CFConv weight images, laid out as the kernels hold them in LDS
    const int prec = d->filter_dtype;
    m->img_bytes = cf_image_bytes(d->D, m->KP, prec);
    const size_t per = m->img_bytes;
    std::vector<unsigned char> hi(per * d->T);
    for (int t = 0; t < d->T; ++t) {
      const float* Wf1 = weights_host + m->off_blk[t];
      const float* cf1 = Wf1 + (size_t)d->Dr * D;
      const float* Wf2 = cf1 + D;
      const float* cf2 = Wf2 + D * D;
      cf_fill_image(d->D, m->KP, prec, d->Dr, Wf1, cf1, Wf2, cf2,
                    (d->rbf_max - d->rbf_min) / (float)(d->Dr - 1), d->r_cut, hi.data() + t * per);
    }
    e = (per == 0) ? hipErrorInvalidValue : hipMalloc(&m->cfimg, hi.size());
    if (e == hipSuccess) e = hipMemcpy(m->cfimg, hi.data(), hi.size(), hipMemcpyHostToDevice);
  }
  if (e == hipSuccess) e = uf_prepare(d->D, m->KP, d->filter_dtype == SN_FILTER_BF16);
  if (e == hipSuccess) {
    // product images of the unfused pipeline
    const int bf16 = d->filter_dtype == SN_FILTER_BF16;
    m->uf_bytes = uf_images(d->D, m->KP, bf16).total;
    std::vector<unsigned char> hu(m->uf_bytes * d->T);
    for (int t = 0; t < d->T; ++t) {
      const float* Wf1 = weights_host + m->off_blk[t];
      const float* Wf2 = Wf1 + (size_t)d->Dr * D + D;
      uf_fill_images(d->D, m->KP, bf16, d->Dr, Wf1, Wf2, hu.data() + t * m->uf_bytes);
    }
    e = hipMalloc(&m->ufimg, hu.size());
    if (e == hipSuccess) e = hipMemcpy(m->ufimg, hu.data(), hu.size(), hipMemcpyHostToDevice);
  }
  if (e == hipSuccess) e = atom_prepare(d->D, d->H, d->filter_dtype);
  if (e == hipSuccess) {
    // atom-wise weight images, laid out as the kernels hold them in LDS
    m->at_upd = atom_image_bytes(d->D, d->D, d->filter_dtype);
    m->at_ro = atom_image_bytes(d->D, d->H, d->filter_dtype);
    std::vector<unsigned char> ha(2 * m->at_upd * d->T + m->at_ro);
    const size_t DD = D * D;
    for (int t = 0; t < d->T; ++t) {
      const float* Wu1 = weights_host + m->off_blk[t] + (size_t)d->Dr * D + D + DD + D;
      const float* cu1 = Wu1 + DD;
      const float* Wu2 = cu1 + D;
      const float* cu2 = Wu2 + DD;
      unsigned char* o = ha.data() + (size_t)t * 2 * m->at_upd;
      atom_fill_image(ATOM_UPDATE_FWD, d->D, d->D, d->filter_dtype, Wu1, cu1, Wu2, cu2, o);
      atom_fill_image(ATOM_UPDATE_BWD, d->D, d->D, d->filter_dtype, Wu1, cu1, Wu2, cu2,
                      o + m->at_upd);
    }
    atom_fill_image(ATOM_READOUT, d->D, d->H, d->filter_dtype, weights_host + m->off_o1,
                    weights_host + m->off_co1,
                    weights_host + m->off_o2, nullptr, ha.data() + (size_t)d->T * 2 * m->at_upd);
    e = (m->at_upd == 0 || m->at_ro == 0) ? hipErrorInvalidValue : hipMalloc(&m->atimg, ha.size());
    if (e == hipSuccess) e = hipMemcpy(m->atimg, ha.data(), ha.size(), hipMemcpyHostToDevice);
  }
  if (e != hipSuccess) {
    sn_model_destroy(m);
    return SN_ERR_HIP;
  }
  *out = m;
  return SN_OK;
}

void sn_model_destroy(sn_model* m) {
  if (!m) return;
  if (m->w) (void)hipFree(m->w);
  if (m->cfimg) (void)hipFree(m->cfimg);
  if (m->atimg) (void)hipFree(m->atimg);
  if (m->ufimg) (void)hipFree(m->ufimg);
  delete m;
}

sn_status sn_workspace_size(const sn_model_desc* d, const sn_system* sys, size_t* bytes) {
  if (!sys || !bytes) return SN_ERR_INVALID_ARG;
  if (!sys_ok(sys)) return SN_ERR_INVALID_ARG;
  if (d && !desc_ok(d)) return SN_ERR_INVALID_ARG;
  *bytes = ws_layout(n_atoms(sys), d ? d->D : 0, d ? d->T : 0, d ? d->H : 0).total;
  return SN_OK;
}

sn_status sn_build_neighbors(const sn_system* sys, const float* pos, float r_list, int32_t* rowptr,
                             int32_t* col, int64_t edge_capacity, int64_t* n_edges_host, void* ws,
                             size_t ws_bytes, hipStream_t s) {
  if (!sys_ok(sys) || !pos || !rowptr || (!col && edge_capacity > 0)) return SN_ERR_INVALID_ARG;
  if (edge_capacity < 0 || edge_capacity > INT32_MAX) return SN_ERR_INVALID_ARG;
  NbrGeom g;
  if (!nbr_geom(sys, r_list, g)) return SN_ERR_INVALID_ARG;
  const WsLayout L = ws_layout(n_atoms(sys), 0, 0, 0);
  sn_status rc = check_ws(ws, ws_bytes, L.total);
  if (rc != SN_OK) return rc;
  char* w = static_cast<char*>(ws);
  hipError_t e = launch_build_neighbors(g, pos, rowptr, col, edge_capacity, w, L, nullptr, 0, s);
  if (e != hipSuccess) return SN_ERR_HIP;
  if (n_edges_host) {
    const DevStatus* st = reinterpret_cast<const DevStatus*>(w + L.status);
    int64_t ne = 0;
    e = hipMemcpyAsync(&ne, &st->last_n_edges, sizeof(int64_t), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return SN_ERR_HIP;
    *n_edges_host = ne;
  }
  return SN_OK;
}

sn_status sn_energy_forces(const sn_model* m, const sn_system* sys, const float* pos,
                           const int32_t* types, const int32_t* rowptr, const int32_t* col,
                           float* energy, float* forces, void* ws, size_t ws_bytes, hipStream_t s) {
  if (!m || !sys_ok(sys) || !pos || !types || !rowptr || !col || !energy || !forces)
    return SN_ERR_INVALID_ARG;
  const WsLayout L = ws_layout(n_atoms(sys), m->desc.D, m->desc.T, m->desc.H);
  sn_status rc = check_ws(ws, ws_bytes, L.total);
  if (rc != SN_OK) return rc;
  return energy_forces_impl(m, sys, pos, types, rowptr, col, energy, forces, static_cast<char*>(ws),
                            s);
}

sn_status sn_energy_forces_noalloc(const sn_model* m, const sn_system* sys, const float* pos,
                                   const int32_t* types, const int32_t* rowptr,
                                   const int32_t* col, float* energy, float* forces,
                                   int64_t* status_dev, hipStream_t s) {
  if (!m || !sys_ok(sys) || !pos || !types || !rowptr || !col || !energy || !forces ||
      !status_dev)
    return SN_ERR_INVALID_ARG;
  const WsLayout L = ws_layout(n_atoms(sys), m->desc.D, m->desc.T, m->desc.H);
  if (L.total > kScratchBytes) return SN_ERR_WORKSPACE;
  char* w = nullptr;
  sn_status rc = scratch_for_current_device(&w);
  if (rc != SN_OK) return rc;
  DevStatus* st = reinterpret_cast<DevStatus*>(w + L.status);
  // the status block starts at zero on every call (a kernel, not a memset:
  // the call may be captured into a graph)
  hipLaunchKernelGGL(k_status_clear, dim3(1), dim3(64), 0, s, st);
  if (hipGetLastError() != hipSuccess) return SN_ERR_HIP;
  rc = energy_forces_impl(m, sys, pos, types, rowptr, col, energy, forces, w, s, nullptr, nullptr,
                          0.f, nullptr, false);
  if (rc != SN_OK) return rc;
  hipLaunchKernelGGL(k_status_copy, dim3(1), dim3(64), 0, s, st, status_dev);
  return hipGetLastError() == hipSuccess ? SN_OK : SN_ERR_HIP;
}

sn_status sn_unfused_workspace_size(const sn_model_desc* d, const sn_system* sys,
                                    int64_t edge_capacity, size_t* bytes) {
  if (!d || !sys || !bytes || !desc_ok(d) || !sys_ok(sys)) return SN_ERR_INVALID_ARG;
  if (edge_capacity < 0 || edge_capacity > INT32_MAX) return SN_ERR_INVALID_ARG;
  const size_t base = ws_layout(n_atoms(sys), d->D, d->T, d->H).total;
  *bytes = uf_layout(base, edge_capacity, d->D, cf_kp(d->Dr, d->filter_dtype),
                     d->T).total;
  return SN_OK;
}

sn_status sn_energy_forces_unfused(const sn_model* m, const sn_system* sys, const float* pos,
                                   const int32_t* types, const int32_t* rowptr,
                                   const int32_t* col, int64_t edge_capacity, int32_t flags,
                                   float* energy, float* forces, void* ws, size_t ws_bytes,
                                   hipStream_t s) {
  if (!m || !sys_ok(sys) || !pos || !types || !rowptr || !col || !energy || !forces)
    return SN_ERR_INVALID_ARG;
  if (edge_capacity < 1 || edge_capacity > INT32_MAX) return SN_ERR_INVALID_ARG;
  if ((flags & ~SN_UNFUSED_ATOMIC) != 0) return SN_ERR_INVALID_ARG;
  if (m->desc.filter_dtype == SN_W16A16 || m->desc.filter_dtype == SN_FILTER_F16X2)
    return SN_ERR_UNSUPPORTED;
  size_t need = 0;
  sn_status rc = sn_unfused_workspace_size(&m->desc, sys, edge_capacity, &need);
  if (rc != SN_OK) return rc;
  rc = check_ws(ws, ws_bytes, need);
  if (rc != SN_OK) return rc;
  const UfMode mode{edge_capacity, (flags & SN_UNFUSED_ATOMIC) ? 1 : 0};
  return energy_forces_impl(m, sys, pos, types, rowptr, col, energy, forces, static_cast<char*>(ws),
                            s, &mode);
}

sn_status sn_md_init(const sn_model* m, const sn_system* sys, const int32_t* types,
                     const sn_md_params* prm, sn_md_state* state, float* energy, void* ws,
                     size_t ws_bytes, hipStream_t s) {
  if (!m || !sys_ok(sys) || !types || !state_ok(state)) return SN_ERR_INVALID_ARG;
  MdSetup su;
  if (!md_setup(m, sys, prm, su)) return SN_ERR_INVALID_ARG;
  NbrGeom g;
  if (!nbr_geom(sys, su.r_list, g)) return SN_ERR_INVALID_ARG;
  const int64_t n = n_atoms(sys);
  const WsLayout L = ws_layout(n, m->desc.D, m->desc.T, m->desc.H);
  sn_status rc = check_ws(ws, ws_bytes, L.total);
  if (rc != SN_OK) return rc;
  char* w = static_cast<char*>(ws);
  DevStatus* st = reinterpret_cast<DevStatus*>(w + L.status);
  float* e_out = energy ? energy : reinterpret_cast<float*>(w + L.eps) + n;
  hipError_t e = hipSuccess;
  if (sys->periodic) e = launch_md_wrap(su.c, n, state->pos, s);
  if (e == hipSuccess) e = launch_md_init_vel(su.c, n, state->vel, s);
  if (e == hipSuccess)
    e = launch_build_neighbors(g, state->pos, state->rowptr, state->col, state->edge_capacity, w, L,
                               nullptr, 0, s);
  const int32_t *rp = nullptr, *cl = nullptr;
  if (e == hipSuccess) e = md_eval_list(m, prm, g, state, w, L, s, rp, cl);
  if (e != hipSuccess) return SN_ERR_HIP;
  // the build's positions are kept by the evaluation's set-up launch
  const BuildMark mark{state->pos, state->pos_at_build, nullptr, 0};
  return energy_forces_impl(m, sys, state->pos, types, rp, cl, e_out, state->forces, w, s, nullptr,
                            nullptr, 0.f, &mark);
}

sn_status sn_md_step(const sn_model* m, const sn_system* sys, const int32_t* types,
                     const sn_md_params* prm, sn_md_state* state, int32_t n_steps, float* energy,
                     void* ws, size_t ws_bytes, hipStream_t s) {
  if (!m || !sys_ok(sys) || !types || !state_ok(state) || n_steps < 0) return SN_ERR_INVALID_ARG;
  MdSetup su;
  if (!md_setup(m, sys, prm, su)) return SN_ERR_INVALID_ARG;
  NbrGeom g;
  if (!nbr_geom(sys, su.r_list, g)) return SN_ERR_INVALID_ARG;
  const int64_t n = n_atoms(sys);
  const WsLayout L = ws_layout(n, m->desc.D, m->desc.T, m->desc.H);
  sn_status rc = check_ws(ws, ws_bytes, L.total);
  if (rc != SN_OK) return rc;
  char* w = static_cast<char*>(ws);
  DevStatus* st = reinterpret_cast<DevStatus*>(w + L.status);
  float* e_out = energy ? energy : reinterpret_cast<float*>(w + L.eps) + n;
  // a displacement flag left by an earlier call (for instance before a restore) must not
  // trigger a rebuild in this one
  if (hipMemsetAsync(&st->rebuild_req, 0, sizeof(int64_t), s) != hipSuccess) return SN_ERR_HIP;
  for (int32_t k = 0; k < n_steps; ++k) {
    const uint64_t step = state->step;
    hipError_t e = launch_md_baoa(su.c, n, step, state->pos, state->vel, state->forces,
                                  state->pos_at_build, st, s);
    if (e != hipSuccess) return SN_ERR_HIP;
    const bool scheduled = ((step + 1) % (uint64_t)prm->rebuild_every) == 0;
    const int64_t* gate = scheduled ? nullptr : &st->rebuild_req;
    const int64_t gval = (int64_t)step + 1;
    e = launch_build_neighbors(g, state->pos, state->rowptr, state->col, state->edge_capacity, w, L,
                               gate, gval, s);
    const int32_t *rp = nullptr, *cl = nullptr;
    if (e == hipSuccess) e = md_eval_list(m, prm, g, state, w, L, s, rp, cl);
    if (e != hipSuccess) return SN_ERR_HIP;
    // the build mark (when this step rebuilt) runs in the evaluation's set-up
    // launch, the closing half-kick B in the launch that sums the forces
    const BuildMark mark{state->pos, state->pos_at_build, gate, gval};
    // the types do not change inside the call: from its second step on, the
    // initial features x0 = Emb[types] in the workspace are still those of
    // the first
    rc = energy_forces_impl(m, sys, state->pos, types, rp, cl, e_out, state->forces, w, s, nullptr,
                            state->vel, su.c.half_kick, &mark, true, k > 0);
    if (rc != SN_OK) return rc;
    state->step = step + 1;
  }
  return SN_OK;
}

sn_status sn_get_device_status(const void* ws, size_t ws_bytes, hipStream_t s, int32_t* status,
                               int64_t* detail, int64_t* n_rebuilds) {
  if (!ws || !status || ws_bytes < sizeof(DevStatus)) return SN_ERR_INVALID_ARG;
  DevStatus h{};
  hipError_t e = hipMemcpyAsync(&h, ws, sizeof(DevStatus), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return SN_ERR_HIP;
  *status = h.status;
  if (detail) *detail = h.detail;
  if (n_rebuilds) *n_rebuilds = h.n_rebuilds;
  return SN_OK;
}

sn_status sn_get_device_counters(const void* ws, size_t ws_bytes, hipStream_t s,
                                 int64_t* evaluations, int64_t* edges_evaluated) {
  if (!ws || !evaluations || !edges_evaluated || ws_bytes < sizeof(DevStatus))
    return SN_ERR_INVALID_ARG;
  DevStatus h{};
  hipError_t e = hipMemcpyAsync(&h, ws, sizeof(DevStatus), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return SN_ERR_HIP;
  *evaluations = h.evaluations;
  *edges_evaluated = h.edges_evaluated;
  return SN_OK;
}

sn_status sn_reset_device_status(void* ws, size_t ws_bytes, hipStream_t s) {
  if (!ws || ws_bytes < sizeof(DevStatus)) return SN_ERR_INVALID_ARG;
  return hip_fail(hipMemsetAsync(ws, 0, sizeof(DevStatus), s));
}

sn_status sn_philox4x64_10(const uint64_t* counters, uint64_t key0, uint64_t key1, uint64_t* out,
                           int64_t n, hipStream_t s) {
  if (n < 0 || (n > 0 && (!counters || !out))) return SN_ERR_INVALID_ARG;
  return hip_fail(launch_philox(counters, key0, key1, out, n, s));
}

sn_status sn_profile_enable(int32_t on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_on = on != 0;
  return SN_OK;
}

sn_status sn_profile_read(int32_t kernel, double* total_ms, int64_t* launches) {
  if (!total_ms || !launches) return SN_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  double sum = 0.0;
  int64_t cnt = 0;
  std::vector<ProfRec> keep;
  for (const ProfRec& r : g_prof_recs) {
    if (r.kernel != kernel) {
      keep.push_back(r);
      continue;
    }
    float ms = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess)
      return SN_ERR_HIP;
    sum += ms;
    ++cnt;
    g_prof_pool.push_back(r.a);
    g_prof_pool.push_back(r.b);
  }
  g_prof_recs.swap(keep);
  *total_ms = sum;
  *launches = cnt;
  return SN_OK;
}

} // extern "C"
