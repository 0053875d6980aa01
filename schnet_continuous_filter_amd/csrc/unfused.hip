// Unfused edge pipeline: the framework-style execution that FlashSchNet's
// ablations take as their starting point. §3.3 lists the bottlenecks (basis
// terms in separate kernels, edge tensors of size E x D written between the
// message-passing steps, contended atomic scatter) and Fig. 2(b) draws this
// pipeline below the fused one; §4.5 "End-to-end integration" names fusion and
// segmented reduction as switches of the ablation.
//
// Every step is its own kernel and leaves its result in an edge tensor:
// distances, Gaussians, envelope, basis B [E][KP], filter pre-activation A,
// its activation, the filter W [E][D] (masked beyond the cutoff), gathered
// sender rows X_src [E][D] and messages M [E][D]. The backward applies the
// chain rule through the same tensors. Aggregation is either an atomic
// scatter-add or a segment sum over receiver rows; the sender-side sums
// (feature gradients, the sender half of the forces) then use the index of
// reverse edges, which on a symmetric list is the source-grouped layout of
// §4.3 "Index construction under dynamic neighbor lists".
//
// The dense products run on MFMA with the weights as the LDS-resident A
// operand (tile16.hpp); everything else streams through HBM.
#include <functional>
#include <type_traits>

#include "tile16.hpp"

namespace sn {

namespace {

constexpr int kUfBlocksPerCu = 8;   // elementwise grids: blocks of kThreads per CU
constexpr int kGemmWaves = 8;       // waves per GEMM work-group
constexpr int kGemmBlocksPerCu = 2;

struct Edges {            // the edge range every kernel reads from the list itself
  const int32_t* rowptr;
  int n;                  // receivers
  int64_t cap;            // edge capacity: edge tensors have this many rows
};

__device__ __forceinline__ int64_t n_edges(const Edges& r) {
  const int64_t e = r.rowptr[r.n];
  return e < r.cap ? e : r.cap;
}

__device__ __forceinline__ int64_t gtid() {
  return (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
}
__device__ __forceinline__ int64_t gstride() { return (int64_t)gridDim.x * blockDim.x; }

__device__ __forceinline__ float uf_min_image(float u, float box, float half) {
  if (u > half) return u - box;
  if (u < -half) return u + box;
  return u;
}

// ------------------------------------------------------------------ indices
__global__ __launch_bounds__(kThreads) void k_uf_capacity(Edges r, DevStatus* st) {
  if (threadIdx.x == 0 && blockIdx.x == 0 && (int64_t)r.rowptr[r.n] > r.cap)
    dev_fail(st, SN_ERR_CAPACITY, r.rowptr[r.n]);
}

// dst[e] = receiver of edge e (the COO receiver index a framework keeps).
__global__ __launch_bounds__(kThreads) void k_uf_dst(Edges r, int32_t* dst) {
  for (int64_t i = gtid(); i < r.n; i += gstride()) {
    int64_t lo = r.rowptr[i], hi = r.rowptr[i + 1];
    if (hi > r.cap) hi = r.cap;
    for (int64_t e = lo; e < hi; ++e) dst[e] = (int32_t)i;
  }
}

// rev[e] = position of the reverse edge (i -> j) of e = (j -> i) in row j,
// by binary search over the ascending senders of that row.
__global__ __launch_bounds__(kThreads) void k_uf_rev(Edges r, const int32_t* col,
                                                     const int32_t* dst, int32_t* rev,
                                                     DevStatus* st) {
  const int64_t E = n_edges(r);
  for (int64_t e = gtid(); e < E; e += gstride()) {
    const int i = dst[e], j = col[e];
    int32_t found = -1;
    if (j >= 0 && j < r.n) {
      int64_t lo = r.rowptr[j], hi = r.rowptr[j + 1];
      if (hi > r.cap) hi = r.cap;
      while (lo < hi) {
        const int64_t mid = (lo + hi) >> 1;
        if (col[mid] < i) lo = mid + 1; else hi = mid;
      }
      if (lo < r.rowptr[j + 1] && lo < r.cap && col[lo] == i) found = (int32_t)lo;
    }
    if (found < 0) dev_fail(st, SN_ERR_INVALID_ARG, e);
    rev[e] = found;
  }
}

// ------------------------------------------------------------------ radial basis, unfused
struct UfBasis {
  int periodic;
  float box, half_box;
  float rbf_min, rbf_step, inv_2s2, inv_s2;   // Gaussian centres mu_k = rbf_min + k step
  float r_cut, pi_over_rc;
  int Dr, KP;
};

// geo[e] = (u, d): u = r_dst - r_src (minimum image), d = |u|.
__global__ __launch_bounds__(kThreads) void k_uf_distance(Edges r, const float* pos,
                                                          const int32_t* dst, const int32_t* col,
                                                          UfBasis b, f32x4* geo) {
  const int64_t E = n_edges(r);
  for (int64_t e = gtid(); e < E; e += gstride()) {
    const int64_t i = dst[e], j = col[e];
    float ux = pos[3 * i] - pos[3 * j];
    float uy = pos[3 * i + 1] - pos[3 * j + 1];
    float uz = pos[3 * i + 2] - pos[3 * j + 2];
    if (b.periodic) {
      ux = uf_min_image(ux, b.box, b.half_box);
      uy = uf_min_image(uy, b.box, b.half_box);
      uz = uf_min_image(uz, b.box, b.half_box);
    }
    geo[e] = f32x4{ux, uy, uz, sqrtf(ux * ux + uy * uy + uz * uz)};
  }
}

// G[e][k] = exp(-(d - mu_k)^2 / (2 sigma^2)) for k < Dr, 0 in the padding.
__global__ __launch_bounds__(kThreads) void k_uf_gauss(Edges r, const f32x4* geo, UfBasis b,
                                                       float* G) {
  const int q = b.KP / 4;
  const int64_t cnt = n_edges(r) * q;
  for (int64_t v = gtid(); v < cnt; v += gstride()) {
    const int64_t e = v / q;
    const int k0 = 4 * (int)(v - e * q);
    const float d = geo[e].w;
    f32x4 o;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int k = k0 + t;
      const float z = d - (b.rbf_min + (float)k * b.rbf_step);
      o[t] = k < b.Dr ? expf(-z * z * b.inv_2s2) : 0.f;
    }
    reinterpret_cast<f32x4*>(G)[v] = o;
  }
}

// C[e] = (cos(pi d / r_c) + 1) / 2 inside the cutoff, else 0; mask[e] = [d < r_c].
__global__ __launch_bounds__(kThreads) void k_uf_cutoff(Edges r, const f32x4* geo, UfBasis b,
                                                        float* C, float* mask) {
  const int64_t E = n_edges(r);
  for (int64_t e = gtid(); e < E; e += gstride()) {
    const float d = geo[e].w;
    const bool in = d < b.r_cut;
    C[e] = in ? 0.5f * (cosf(b.pi_over_rc * d) + 1.f) : 0.f;
    mask[e] = in ? 1.f : 0.f;
  }
}

// X[e][:] *= s[e] (row width W, a multiple of 4), in place.
__global__ __launch_bounds__(kThreads) void k_uf_rowscale(Edges r, float* X, const float* s,
                                                          int W) {
  const int q = W / 4;
  const int64_t cnt = n_edges(r) * q;
  for (int64_t v = gtid(); v < cnt; v += gstride()) {
    f32x4* p = reinterpret_cast<f32x4*>(X) + v;
    *p = *p * s[v / q];
  }
}

// ------------------------------------------------------------------ dense products
// Y[e][:] = X[e][:] M (+ bias) for 16-edge tiles; M [K][N] is an output-major
// image (uf_fill_images) staged once per work-group into LDS.
template <int K, int N, int PR>
__global__ __launch_bounds__(64 * kGemmWaves) void k_uf_gemm(Edges r, const float* X,
                                                            const void* img, const float* bias,
                                                            float* Y) {
  constexpr int IMG = N * K * (PR != PREC_F32 ? 2 : 4);
  extern __shared__ __align__(16) unsigned char lds[];
  stage_lds<IMG, 64 * kGemmWaves>(img, lds);
  __syncthreads();
  const int lane = threadIdx.x & 63, e = lane & 15, g = lane >> 4;
  const int wave = uni((int)threadIdx.x >> 6);
  const int64_t E = n_edges(r);
  const int64_t ntiles = (E + 15) / 16;
  for (int64_t t = (int64_t)blockIdx.x * kGemmWaves + wave; t < ntiles;
       t += (int64_t)gridDim.x * kGemmWaves) {
    const int64_t row = t * 16 + e;
    const bool ok = row < E;
    f32x4 S[K / 16];
    const float* xr = X + row * K + 4 * g;
#pragma unroll
    for (int c = 0; c < K / 16; ++c)
      S[c] = ok ? *reinterpret_cast<const f32x4*>(xr + 16 * c) : f32x4{};
    f32x4 out[N / 16];
    gemm_om<K, N, PR>(out, S, lds, lane);
    if (ok) {
      float* yr = Y + row * N + 4 * g;
#pragma unroll
      for (int nb = 0; nb < N / 16; ++nb) {
        f32x4 v = out[nb];
        if (bias) v += *reinterpret_cast<const f32x4*>(bias + 16 * nb + 4 * g);
        *reinterpret_cast<f32x4*>(yr + 16 * nb) = v;
      }
    }
  }
}

// ------------------------------------------------------------------ elementwise over E x W
// S = ssp(A) = ln(1 + e^A) - ln 2, computed as max(A, 0) + log1p(e^-|A|) - ln 2.
__global__ __launch_bounds__(kThreads) void k_uf_ssp(Edges r, const float* A, float* S, int W) {
  const int64_t cnt = n_edges(r) * (W / 4);
  for (int64_t v = gtid(); v < cnt; v += gstride()) {
    const f32x4 a = reinterpret_cast<const f32x4*>(A)[v];
    f32x4 o;
#pragma unroll
    for (int t = 0; t < 4; ++t) o[t] = fmaxf(a[t], 0.f) + log1pf(expf(-fabsf(a[t]))) - LN2F;
    reinterpret_cast<f32x4*>(S)[v] = o;
  }
}

// G *= sigmoid(A), in place (the derivative of ssp).
__global__ __launch_bounds__(kThreads) void k_uf_sigmul(Edges r, float* G, const float* A, int W) {
  const int64_t cnt = n_edges(r) * (W / 4);
  for (int64_t v = gtid(); v < cnt; v += gstride()) {
    const f32x4 a = reinterpret_cast<const f32x4*>(A)[v];
    f32x4 o = reinterpret_cast<f32x4*>(G)[v];
#pragma unroll
    for (int t = 0; t < 4; ++t) o[t] = o[t] / (1.f + expf(-a[t]));
    reinterpret_cast<f32x4*>(G)[v] = o;
  }
}

// out[e][:] = x[idx[e]][:] (row gather of per-atom features).
__global__ __launch_bounds__(kThreads) void k_uf_gather(Edges r, const float* x,
                                                        const int32_t* idx, int W, float* out) {
  const int q = W / 4;
  const int64_t cnt = n_edges(r) * q;
  for (int64_t v = gtid(); v < cnt; v += gstride()) {
    const int64_t e = v / q;
    const int c = (int)(v - e * q);
    reinterpret_cast<f32x4*>(out)[v] =
        reinterpret_cast<const f32x4*>(x)[(int64_t)idx[e] * q + c];
  }
}

// out = a * b (* s[e] per row when s is not null).
__global__ __launch_bounds__(kThreads) void k_uf_mul(Edges r, const float* a, const float* b,
                                                     const float* s, int W, float* out) {
  const int q = W / 4;
  const int64_t cnt = n_edges(r) * q;
  for (int64_t v = gtid(); v < cnt; v += gstride()) {
    f32x4 o = reinterpret_cast<const f32x4*>(a)[v] * reinterpret_cast<const f32x4*>(b)[v];
    if (s) o = o * s[v / q];
    reinterpret_cast<f32x4*>(out)[v] = o;
  }
}

// ------------------------------------------------------------------ aggregation
// h[idx[e]][:] += M[e][:] by atomic adds (hardware fp32 add in L2).
__global__ __launch_bounds__(kThreads) void k_uf_scatter(Edges r, const float* M,
                                                         const int32_t* idx, int W, float* h) {
  const int q = W / 4;
  const int64_t cnt = n_edges(r) * q;
  for (int64_t v = gtid(); v < cnt; v += gstride()) {
    const int64_t e = v / q;
    const int c = (int)(v - e * q);
    const f32x4 m = reinterpret_cast<const f32x4*>(M)[v];
    float* o = h + (int64_t)idx[e] * W + 4 * c;
#pragma unroll
    for (int t = 0; t < 4; ++t) unsafeAtomicAdd(o + t, m[t]);
  }
}

// h[i][:] = sum over e in row i of M[e][:] (or of M[rev[e]][:]), ascending e:
// one wave per receiver, W / 64 features per lane, one store per row.
template <int W>
__global__ __launch_bounds__(kThreads) void k_uf_segsum(Edges r, const float* M,
                                                        const int32_t* rev, float* h) {
  constexpr int PL = W / 64;
  const int lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (i >= r.n) return;
  int64_t lo = r.rowptr[i], hi = r.rowptr[i + 1];
  if (hi > r.cap) hi = r.cap;
  float acc[PL];
#pragma unroll
  for (int t = 0; t < PL; ++t) acc[t] = 0.f;
  for (int64_t e = lo; e < hi; ++e) {
    const int64_t src = rev ? (int64_t)rev[e] : e;
    if (src < 0) continue;
    const float* m = M + src * W + PL * lane;
#pragma unroll
    for (int t = 0; t < PL; ++t) acc[t] += m[t];
  }
#pragma unroll
  for (int t = 0; t < PL; ++t) h[i * W + PL * lane + t] = acc[t];
}

// ------------------------------------------------------------------ distance gradient and forces
// gd[e] = sum_k gB[e][k] d b~_k / dd with b~_k = g_k C: KP / 4 lanes per edge.
__global__ __launch_bounds__(kThreads) void k_uf_gd(Edges r, const float* gB, const f32x4* geo,
                                                    UfBasis b, float* gd) {
  const int lpe = b.KP / 4;                 // 8 or 16 lanes per edge
  const int64_t E = n_edges(r);
  const int64_t cnt = E * lpe;
  const int64_t span = (cnt + 63) / 64 * 64;  // whole waves take part in the shuffles
  for (int64_t v = gtid(); v < span; v += gstride()) {
    float part = 0.f;
    if (v < cnt) {
      const int64_t e = v / lpe;
      const int k0 = 4 * (int)(v - e * lpe);
      const float d = geo[e].w;
      const bool in = d < b.r_cut;
      const float C = in ? 0.5f * (cosf(b.pi_over_rc * d) + 1.f) : 0.f;
      const float Cp = in ? -0.5f * b.pi_over_rc * sinf(b.pi_over_rc * d) : 0.f;
      const f32x4 gb = reinterpret_cast<const f32x4*>(gB)[v];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int k = k0 + t;
        if (k < b.Dr) {
          const float z = d - (b.rbf_min + (float)k * b.rbf_step);
          const float gk = expf(-z * z * b.inv_2s2);
          part += gb[t] * gk * (Cp - C * z * b.inv_s2);
        }
      }
    }
    for (int o = lpe / 2; o > 0; o >>= 1) part += __shfl_xor(part, o, 64);
    if (v < cnt && (v % lpe) == 0) gd[v / lpe] = part;
  }
}

// dE/dr[dst] += gd u / d and dE/dr[src] -= gd u / d, by atomic adds.
__global__ __launch_bounds__(kThreads) void k_uf_force_atomic(Edges r, const float* gd,
                                                              const f32x4* geo,
                                                              const int32_t* dst,
                                                              const int32_t* col, float* dEdr) {
  const int64_t E = n_edges(r);
  for (int64_t e = gtid(); e < E; e += gstride()) {
    const f32x4 u = geo[e];
    const float s = u.w > 0.f ? gd[e] / u.w : 0.f;
    float* a = dEdr + 3 * (int64_t)dst[e];
    float* c = dEdr + 3 * (int64_t)col[e];
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      unsafeAtomicAdd(a + t, s * u[t]);
      unsafeAtomicAdd(c + t, -s * u[t]);
    }
  }
}

// dE/dr[i] += sum over e in row i of (gd[e] + gd[rev[e]]) u_e / d_e: the
// reverse edge carries the sender half of i's pairs (u_rev = -u_e).
__global__ __launch_bounds__(kThreads) void k_uf_force_seg(Edges r, const float* gd,
                                                           const f32x4* geo, const int32_t* rev,
                                                           float* dEdr) {
  for (int64_t i = gtid(); i < r.n; i += gstride()) {
    int64_t lo = r.rowptr[i], hi = r.rowptr[i + 1];
    if (hi > r.cap) hi = r.cap;
    float fx = 0.f, fy = 0.f, fz = 0.f;
    for (int64_t e = lo; e < hi; ++e) {
      const f32x4 u = geo[e];
      const int32_t re = rev[e];
      const float g = gd[e] + (re >= 0 ? gd[re] : 0.f);
      const float s = u.w > 0.f ? g / u.w : 0.f;
      fx += s * u.x;
      fy += s * u.y;
      fz += s * u.z;
    }
    dEdr[3 * i] += fx;
    dEdr[3 * i + 1] += fy;
    dEdr[3 * i + 2] += fz;
  }
}

__global__ __launch_bounds__(kThreads) void k_uf_fill(float* p, int64_t n, float v) {
  for (int64_t i = gtid(); i < n; i += gstride()) p[i] = v;
}

// ------------------------------------------------------------------ host side
void om_image_k(int K, int N, int bf16, int Kin, int Nin,
                const std::function<float(int, int)>& m, unsigned char* out) {
  auto go = [&](auto kk) {
    constexpr int KK = decltype(kk)::value;
    if (bf16) om_image<KK, PREC_BF16>(N, Kin, Nin, m, out, nullptr);
    else om_image<KK, PREC_F32>(N, Kin, Nin, m, out, nullptr);
  };
  switch (K) {
    case 32: go(std::integral_constant<int, 32>{}); break;
    case 64: go(std::integral_constant<int, 64>{}); break;
    default: go(std::integral_constant<int, 128>{}); break;
  }
}

size_t img_bytes(int K, int N, int bf16) { return (size_t)K * N * (bf16 ? 2 : 4); }

template <int K, int N, int PR>
hipError_t gemm_prepare() {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&k_uf_gemm<K, N, PR>),
                             hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)img_bytes(K, N, PR != PREC_F32));
}

template <int K, int N, int PR>
hipError_t gemm_launch(Edges r, const float* X, const void* img, const float* bias, float* Y,
                       int n_cu, hipStream_t s) {
  hipLaunchKernelGGL((k_uf_gemm<K, N, PR>), dim3(n_cu * kGemmBlocksPerCu),
                     dim3(64 * kGemmWaves), img_bytes(K, N, PR != PREC_F32), s, r, X, img, bias,
                     Y);
  return hipGetLastError();
}

// The (K, N) shapes of the four products: (KP, D), (D, D), (D, D), (D, KP).
template <int PR>
hipError_t gemm_dispatch(int K, int N, Edges r, const float* X, const void* img,
                         const float* bias, float* Y, int n_cu, hipStream_t s, bool prepare) {
#define SN_UF_CASE(KK, NN)                                                 \
  if (K == KK && N == NN)                                                  \
    return prepare ? gemm_prepare<KK, NN, PR>()                            \
                   : gemm_launch<KK, NN, PR>(r, X, img, bias, Y, n_cu, s);
  SN_UF_CASE(32, 64) SN_UF_CASE(32, 128) SN_UF_CASE(64, 64) SN_UF_CASE(64, 128)
  SN_UF_CASE(128, 128) SN_UF_CASE(64, 32) SN_UF_CASE(128, 32) SN_UF_CASE(128, 64)
#undef SN_UF_CASE
  return hipErrorInvalidValue;
}

hipError_t gemm(int K, int N, int bf16, Edges r, const float* X, const void* img,
                const float* bias, float* Y, int n_cu, hipStream_t s) {
  return bf16 ? gemm_dispatch<PREC_BF16>(K, N, r, X, img, bias, Y, n_cu, s, false)
              : gemm_dispatch<PREC_F32>(K, N, r, X, img, bias, Y, n_cu, s, false);
}

} // namespace

// Offsets of the four product images of one block inside its image.
UfImages uf_images(int D, int KP, int bf16) {
  UfImages m{};
  m.g1 = 0;
  m.g2 = m.g1 + img_bytes(KP, D, bf16);
  m.g3 = m.g2 + img_bytes(D, D, bf16);
  m.g4 = m.g3 + img_bytes(D, D, bf16);
  m.total = m.g4 + img_bytes(D, KP, bf16);
  return m;
}

void uf_fill_images(int D, int KP, int bf16, int Dr, const float* Wf1, const float* Wf2,
                    unsigned char* out) {
  const UfImages m = uf_images(D, KP, bf16);
  // A = B Wf1:   (k, n) = Wf1[k][n], k < Dr
  om_image_k(KP, D, bf16, Dr, D, [&](int k, int n) { return Wf1[(size_t)k * D + n]; }, out + m.g1);
  // W = S Wf2
  om_image_k(D, D, bf16, D, D, [&](int k, int n) { return Wf2[(size_t)k * D + n]; }, out + m.g2);
  // dS = dW Wf2^T
  om_image_k(D, D, bf16, D, D, [&](int k, int n) { return Wf2[(size_t)n * D + k]; }, out + m.g3);
  // dB = dA Wf1^T:  (k, n) = Wf1[n][k], n < Dr
  om_image_k(D, KP, bf16, D, Dr, [&](int k, int n) { return Wf1[(size_t)n * D + k]; },
             out + m.g4);
}

hipError_t uf_prepare(int D, int KP, int bf16) {
  const int shapes[4][2] = {{KP, D}, {D, D}, {D, D}, {D, KP}};
  for (auto& sh : shapes) {
    const Edges r{nullptr, 0, 0};
    const hipError_t e =
        bf16 ? gemm_dispatch<PREC_BF16>(sh[0], sh[1], r, nullptr, nullptr, nullptr, nullptr, 0, 0,
                                        true)
             : gemm_dispatch<PREC_F32>(sh[0], sh[1], r, nullptr, nullptr, nullptr, nullptr, 0, 0,
                                       true);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_unfused(const UfArgs& a, hipStream_t s) {
  const Edges r{a.rowptr, a.n_atoms, a.cap};
  const int D = a.D, KP = a.KP, bf16 = a.bf16;
  const dim3 grid(a.n_cu * kUfBlocksPerCu), blk(kThreads);
  const dim3 wave_grid((unsigned)((a.n_atoms + kThreads / 64 - 1) / (kThreads / 64)));
  const UfBasis b{a.periodic, a.box, 0.5f * a.box, a.rbf_min, a.rbf_step,
                  (float)(0.5 / ((double)a.rbf_step * a.rbf_step)),
                  (float)(1.0 / ((double)a.rbf_step * a.rbf_step)), a.r_cut,
                  (float)(M_PI / (double)a.r_cut), a.Dr, KP};
  hipError_t e;
  auto seg = [&](const float* M, const int32_t* rev, float* h) {
    if (D == 128) hipLaunchKernelGGL(k_uf_segsum<128>, wave_grid, blk, 0, s, r, M, rev, h);
    else hipLaunchKernelGGL(k_uf_segsum<64>, wave_grid, blk, 0, s, r, M, rev, h);
    return hipGetLastError();
  };

  switch (a.phase) {
    case UF_EDGES: {
      hipLaunchKernelGGL(k_uf_capacity, dim3(1), dim3(64), 0, s, r, a.st);
      hipLaunchKernelGGL(k_uf_dst, dim3((a.n_atoms + kThreads - 1) / kThreads), blk, 0, s, r,
                         a.dst);
      if (!a.atomic)
        hipLaunchKernelGGL(k_uf_rev, grid, blk, 0, s, r, a.col, a.dst, a.rev, a.st);
      hipLaunchKernelGGL(k_uf_distance, grid, blk, 0, s, r, a.pos, a.dst, a.col, b, a.geo);
      hipLaunchKernelGGL(k_uf_gauss, grid, blk, 0, s, r, a.geo, b, a.B);
      hipLaunchKernelGGL(k_uf_cutoff, grid, blk, 0, s, r, a.geo, b, a.C, a.mask);
      hipLaunchKernelGGL(k_uf_rowscale, grid, blk, 0, s, r, a.B, a.C, KP);
      hipLaunchKernelGGL(k_uf_fill, grid, blk, 0, s, a.dEdr, (int64_t)a.n_atoms * 3, 0.f);
      return hipGetLastError();
    }
    case UF_FORWARD: {
      const unsigned char* img = static_cast<const unsigned char*>(a.img);
      const UfImages im = uf_images(D, KP, bf16);
      // A = B Wf1 + cf1 ; S = ssp(A) ; W = (S Wf2 + cf2) * mask
      if ((e = gemm(KP, D, bf16, r, a.B, img + im.g1, a.cf1, a.A, a.n_cu, s)) != hipSuccess)
        return e;
      hipLaunchKernelGGL(k_uf_ssp, grid, blk, 0, s, r, a.A, a.buf0, D);
      if ((e = gemm(D, D, bf16, r, a.buf0, img + im.g2, a.cf2, a.W, a.n_cu, s)) != hipSuccess)
        return e;
      hipLaunchKernelGGL(k_uf_rowscale, grid, blk, 0, s, r, a.W, a.mask, D);
      // X_src = x[src] ; M = X_src * W ; h = sum over receivers
      hipLaunchKernelGGL(k_uf_gather, grid, blk, 0, s, r, a.x, a.col, D, a.Xs);
      hipLaunchKernelGGL(k_uf_mul, grid, blk, 0, s, r, a.Xs, a.W, nullptr, D, a.buf0);
      if (a.atomic) {
        hipLaunchKernelGGL(k_uf_fill, grid, blk, 0, s, a.h, (int64_t)a.n_atoms * D, 0.f);
        hipLaunchKernelGGL(k_uf_scatter, grid, blk, 0, s, r, a.buf0, a.dst, D, a.h);
        return hipGetLastError();
      }
      return seg(a.buf0, nullptr, a.h);
    }
    case UF_BACKWARD: {
      const unsigned char* img = static_cast<const unsigned char*>(a.img);
      const UfImages im = uf_images(D, KP, bf16);
      // dM = gh[dst] ; dX_src = dM * W -> sender sums q ; dW = dM * X_src * mask
      hipLaunchKernelGGL(k_uf_gather, grid, blk, 0, s, r, a.gh, a.dst, D, a.buf0);
      if (a.q) {
        hipLaunchKernelGGL(k_uf_mul, grid, blk, 0, s, r, a.buf0, a.W, nullptr, D, a.buf1);
        if (a.atomic) {
          hipLaunchKernelGGL(k_uf_fill, grid, blk, 0, s, a.q, (int64_t)a.n_atoms * D, 0.f);
          hipLaunchKernelGGL(k_uf_scatter, grid, blk, 0, s, r, a.buf1, a.col, D, a.q);
        } else if ((e = seg(a.buf1, a.rev, a.q)) != hipSuccess) {
          return e;
        }
      }
      hipLaunchKernelGGL(k_uf_mul, grid, blk, 0, s, r, a.buf0, a.Xs, a.mask, D, a.buf2);
      // dS = dW Wf2^T ; dA = dS * sigmoid(A) ; dB = dA Wf1^T
      if ((e = gemm(D, D, bf16, r, a.buf2, img + im.g3, nullptr, a.buf1, a.n_cu, s)) !=
          hipSuccess)
        return e;
      hipLaunchKernelGGL(k_uf_sigmul, grid, blk, 0, s, r, a.buf1, a.A, D);
      if ((e = gemm(D, KP, bf16, r, a.buf1, img + im.g4, nullptr, a.gB, a.n_cu, s)) != hipSuccess)
        return e;
      // dE/dd, then dE/dr on both ends of every edge
      hipLaunchKernelGGL(k_uf_gd, grid, blk, 0, s, r, a.gB, a.geo, b, a.gd);
      if (a.atomic)
        hipLaunchKernelGGL(k_uf_force_atomic, grid, blk, 0, s, r, a.gd, a.geo, a.dst, a.col,
                           a.dEdr);
      else
        hipLaunchKernelGGL(k_uf_force_seg, grid, blk, 0, s, r, a.gd, a.geo, a.rev, a.dEdr);
      return hipGetLastError();
    }
  }
  return hipErrorInvalidValue;
}

} // namespace sn
