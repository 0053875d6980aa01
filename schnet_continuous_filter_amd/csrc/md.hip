// Langevin dynamics over batched replicas (BAOAB) and its noise generator.
//
// FlashSchNet §5.1 "Experimental setting" runs Langevin dynamics at 300 K over
// parallel replicas, and §4.5 "End-to-end integration" lists the per-step work
// (rebuild the neighbour list and its segment index, evaluate energy and
// forces). The page names no integrator; these kernels implement the BAOAB
// splitting of Leimkuhler and Matthews (2013). All replicas advance in one
// launch: one thread per atom.
//
// Noise: Philox4x64-10 (Salmon, Moraes, Dror and Shaw, "Parallel random
// numbers: as easy as 1, 2, 3", SC'11): ten rounds of two 64x64->128-bit
// multiplies with the published multipliers and Weyl key increments. Counter
// (atom, step, stream, 0), key (seed, 0); words -> uniforms
// ((w >> 11) + 0.5) 2^-53 -> Box-Muller in double.
#include "common.hpp"

namespace sn {

__device__ __forceinline__ void philox_round(uint64_t c[4], uint64_t k0, uint64_t k1) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t hi0 = __umul64hi(M0, c[0]), lo0 = M0 * c[0];
  const uint64_t hi1 = __umul64hi(M1, c[2]), lo1 = M1 * c[2];
  const uint64_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
  c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
}

__device__ __forceinline__ void philox4x64_10(uint64_t c[4], uint64_t k0, uint64_t k1) {
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    philox_round(c, k0, k1);
    k0 += W0;
    k1 += W1;
  }
}

// Three standard normals for (atom, step, stream).
__device__ __forceinline__ void normals3(uint64_t seed, uint64_t step, uint64_t stream,
                                         uint64_t atom, double z[3]) {
  uint64_t c[4] = {atom, step, stream, 0};
  philox4x64_10(c, seed, 0);
  double u[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) u[k] = ((double)(c[k] >> 11) + 0.5) * 0x1.0p-53;
  const double two_pi = 2.0 * 3.14159265358979323846;
  const double r01 = sqrt(-2.0 * log(u[0]));
  const double r23 = sqrt(-2.0 * log(u[2]));
  double s1, c1;
  sincos(two_pi * u[1], &s1, &c1);
  z[0] = r01 * c1;
  z[1] = r01 * s1;
  z[2] = r23 * cos(two_pi * u[3]);
}

__device__ __forceinline__ float wrap(float x, float box) {
  float y = x - box * floorf(x / box);
  return (y >= box || y < 0.f) ? 0.f : y;
}

__global__ __launch_bounds__(kThreads) void k_md_init_vel(MdCoef c, int64_t n, float* vel) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= n) return;
  double z[3];
  normals3(c.seed, 0, 1, (uint64_t)i, z);
  for (int k = 0; k < 3; ++k) vel[3 * i + k] = c.sigma_v * (float)z[k];
}

__global__ __launch_bounds__(kThreads) void k_md_wrap(MdCoef c, int64_t n, float* pos) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= n) return;
  for (int k = 0; k < 3; ++k) pos[3 * i + k] = wrap(pos[3 * i + k], c.box);
}

// B A O A for step `step`; flags a rebuild when an atom moved more than skin/2
// since the last build, and reports an atom whose new position or velocity is
// not finite (detail -(1 + atom)): its edges would otherwise vanish from the
// next list without a trace.
__global__ __launch_bounds__(kThreads) void k_md_baoa(MdCoef c, int64_t n, uint64_t step,
                                                      float* pos, float* vel,
                                                      const float* forces,
                                                      const float* pos_at_build, DevStatus* st) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= n) return;
  double z[3];
  normals3(c.seed, step, 0, (uint64_t)i, z);
  float d2 = 0.f;
  bool finite = true;
  for (int k = 0; k < 3; ++k) {
    float v = vel[3 * i + k] + c.half_kick * forces[3 * i + k];
    float r = pos[3 * i + k] + c.half_dt * v;
    v = c.c1 * v + c.c2 * (float)z[k];
    r = r + c.half_dt * v;
    float dd;
    if (c.periodic) {
      r = wrap(r, c.box);
      dd = r - pos_at_build[3 * i + k];
      dd -= c.box * rintf(dd / c.box);
    } else {
      dd = r - pos_at_build[3 * i + k];
    }
    d2 += dd * dd;
    finite = finite && isfinite(r) && isfinite(v);
    vel[3 * i + k] = v;
    pos[3 * i + k] = r;
  }
  if (!finite) dev_fail(st, SN_ERR_NONFINITE, -1 - i);
  if (d2 > c.half_skin2) st->rebuild_req = (int64_t)step + 1;
}

__global__ __launch_bounds__(kThreads) void k_philox(const uint64_t* ctr, uint64_t k0, uint64_t k1,
                                                     uint64_t* out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= n) return;
  uint64_t c[4] = {ctr[4 * i], ctr[4 * i + 1], ctr[4 * i + 2], ctr[4 * i + 3]};
  philox4x64_10(c, k0, k1);
  for (int k = 0; k < 4; ++k) out[4 * i + k] = c[k];
}

static dim3 grid_for(int64_t n) { return dim3((unsigned)((n + kThreads - 1) / kThreads)); }

hipError_t launch_md_init_vel(const MdCoef& c, int64_t n, float* vel, hipStream_t s) {
  hipLaunchKernelGGL(k_md_init_vel, grid_for(n), dim3(kThreads), 0, s, c, n, vel);
  return hipGetLastError();
}
hipError_t launch_md_wrap(const MdCoef& c, int64_t n, float* pos, hipStream_t s) {
  hipLaunchKernelGGL(k_md_wrap, grid_for(n), dim3(kThreads), 0, s, c, n, pos);
  return hipGetLastError();
}
hipError_t launch_md_baoa(const MdCoef& c, int64_t n, uint64_t step, float* pos, float* vel,
                          const float* forces, const float* pos_at_build, DevStatus* st,
                          hipStream_t s) {
  hipLaunchKernelGGL(k_md_baoa, grid_for(n), dim3(kThreads), 0, s, c, n, step, pos, vel, forces,
                     pos_at_build, st);
  return hipGetLastError();
}
hipError_t launch_philox(const uint64_t* ctr, uint64_t k0, uint64_t k1, uint64_t* out, int64_t n,
                         hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_philox, grid_for(n), dim3(kThreads), 0, s, ctr, k0, k1, out, n);
  return hipGetLastError();
}

} // namespace sn
