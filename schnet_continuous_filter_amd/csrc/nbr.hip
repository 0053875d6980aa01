// Neighbour list: directed edges within a radius, grouped by receiver (CSR).
//
// FlashSchNet, §3.2 "Building the neighbor list" defines the edge set (edge
// j = src -> i = dst within the cutoff) and §4.3 "Index construction under
// dynamic neighbor lists" groups edges into one contiguous segment per
// destination by a bucket sort. Here the segments are produced directly:
// count per receiver -> exclusive scan -> fill, with senders ascending.
//
// Membership is decided in IEEE double arithmetic without contraction on the
// float inputs (see pair_in), so the list is identical to the one a host
// computes with the same sequence of operations, and symmetric.
//
// Two search modes:
//  * all pairs inside each replica (chains and small boxes), one wave per
//    receiver with ballot compaction; senders ascend, so rows come out sorted;
//  * a cell list for one large system: a periodic cube, or an open system
//    whose bounding box the device finds first; cells of edge >= r_list,
//    27-cell search (without wrap-around for open systems), then a per-row
//    rank sort in LDS.
#include "common.hpp"

namespace sn {

// Exact membership test for the edge j -> i.
__device__ __forceinline__ bool pair_in(float xi, float yi, float zi, float xj, float yj, float zj,
                                        int periodic, double L, double half, double r2) {
#pragma clang fp contract(off)
  double dx = (double)xj - (double)xi;
  double dy = (double)yj - (double)yi;
  double dz = (double)zj - (double)zi;
  if (periodic) {
    if (dx > half) dx = dx - L; else if (dx < -half) dx = dx + L;
    if (dy > half) dy = dy - L; else if (dy < -half) dy = dy + L;
    if (dz > half) dz = dz - L; else if (dz < -half) dz = dz + L;
  }
  double sx = dx * dx;
  double sy = dy * dy;
  double sz = dz * dz;
  double s = (sx + sy) + sz;
  return s < r2;
}

// A non-finite position fails every membership test, so its atom would
// silently lose its edges: it is reported instead (detail -(1 + atom)).
__device__ __forceinline__ void check_position(DevStatus* st, int64_t atom, float x, float y,
                                               float z) {
  if (!(isfinite(x) && isfinite(y) && isfinite(z))) dev_fail(st, SN_ERR_NONFINITE, -1 - atom);
}

#define SN_GATE                                   \
  if (gate != nullptr && *gate != gate_val) return;

// ------------------------------------------------------------------ scan
// Exclusive scan of one value per thread over an NT-thread block.
template <int NT = kThreads>
__device__ inline int64_t block_exclusive_scan(int64_t v, int64_t* smem, int64_t* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int64_t x = v;
  for (int off = 1; off < 64; off <<= 1) {
    int64_t y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) smem[wave] = x;
  __syncthreads();
  int64_t wave_off = 0, tot = 0;
  for (int w = 0; w < NT / 64; ++w) {
    if (w < wave) wave_off += smem[w];
    tot += smem[w];
  }
  __syncthreads();
  *total = tot;
  return wave_off + x - v;
}

__global__ __launch_bounds__(kThreads) void k_scan_local(int32_t* a, int64_t n, int64_t* blocks,
                                                         const int64_t* gate, int64_t gate_val) {
  SN_GATE
  __shared__ int64_t smem[kThreads / 64];
  const int64_t base = (int64_t)blockIdx.x * kScanChunk + 4 * threadIdx.x;
  int64_t v[4], s = 0;
  for (int q = 0; q < 4; ++q) {
    v[q] = (base + q < n) ? a[base + q] : 0;
    s += v[q];
  }
  int64_t tot;
  int64_t ex = block_exclusive_scan(s, smem, &tot);
  for (int q = 0; q < 4; ++q) {
    if (base + q < n) a[base + q] = (int32_t)ex;  // block-local prefix (block sums < 2^31)
    ex += v[q];
  }
  if (threadIdx.x == 0) blocks[blockIdx.x] = tot;
}

__global__ __launch_bounds__(kThreads) void k_scan_top(int64_t* blocks, int64_t nblk, DevStatus* st,
                                                       int64_t capacity, const int64_t* gate,
                                                       int64_t gate_val) {
  SN_GATE
  __shared__ int64_t smem[kThreads / 64];
  int64_t running = 0;
  for (int64_t c0 = 0; c0 < nblk; c0 += 4 * kThreads) {
    const int64_t base = c0 + 4 * threadIdx.x;
    int64_t v[4], s = 0;
    for (int q = 0; q < 4; ++q) {
      v[q] = (base + q < nblk) ? blocks[base + q] : 0;
      s += v[q];
    }
    int64_t tot;
    int64_t ex = block_exclusive_scan(s, smem, &tot);
    for (int q = 0; q < 4; ++q) {
      if (base + q < nblk) blocks[base + q] = running + ex;
      ex += v[q];
    }
    running += tot;
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    blocks[nblk] = running;
    if (capacity >= 0) {
      const int ovf = running > capacity;
      st->last_n_edges = running;
      st->overflow = ovf;
      if (ovf) dev_fail(st, SN_ERR_CAPACITY, running);
    }
  }
}

__global__ __launch_bounds__(kThreads) void k_scan_add(int32_t* a, int64_t n, const int64_t* blocks,
                                                       int64_t nblk, int64_t capacity,
                                                       const int64_t* gate, int64_t gate_val) {
  SN_GATE
  const int64_t total = blocks[nblk];
  const bool ovf = capacity >= 0 && total > capacity;
  const int64_t off = blocks[blockIdx.x];
  const int64_t base = (int64_t)blockIdx.x * kScanChunk + 4 * threadIdx.x;
  for (int q = 0; q < 4; ++q)
    if (base + q < n) a[base + q] = ovf ? 0 : (int32_t)(a[base + q] + off);
  if (blockIdx.x == 0 && threadIdx.x == 0) a[n] = ovf ? 0 : (int32_t)total;
}

// Inclusive scan over the 64 lanes of a wave on DPP lane moves: shifts by 1,
// 2, 4 and 8 inside each row of 16 lanes (lanes without a source add 0),
// then lane 15 of rows 0 and 2 added to rows 1 and 3, then lane 31 added to
// rows 2 and 3.
__device__ __forceinline__ int32_t wave_inclusive_scan(int32_t x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31
  return x;
}

// Lists of up to 32,768 rows are scanned by one block of kScan1Threads
// threads in one launch. Wave w owns the contiguous run [w 64 Q, (w + 1) 64 Q);
// its Q loads of 64 consecutive counts (one per lane, bounded: reads past n
// give 0) are all issued before the first is used; the wave scans them in
// order, carrying its running total, and one block scan of the sixteen wave
// totals gives each wave its offset.
constexpr int kScan1Threads = 1024;
constexpr int64_t kScan1Max = 32768;
template <int Q>
__global__ __launch_bounds__(kScan1Threads) void k_scan_single(int32_t* a, int64_t n,
                                                              DevStatus* st, int64_t capacity,
                                                              const int64_t* gate,
                                                              int64_t gate_val) {
  SN_GATE
  __shared__ int64_t smem[kScan1Threads / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc(a, (short)0, (int)(n * 4), 0x00020000);
  const uint32_t base = (uint32_t)(wave * 64 * Q + lane);
  int32_t v[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q)
    v[q] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(ra, (base + 64u * q) * 4u, 0, 0);
  // exclusive prefixes within each group of 64, chained over the groups in order
  int64_t carry = 0;
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int32_t x = wave_inclusive_scan(v[q]);
    const int32_t wtot = __builtin_amdgcn_readlane(x, 63);
    v[q] = (int32_t)(carry + (x - v[q]));
    carry += wtot;
  }
  int64_t tot;
  const int64_t off = block_exclusive_scan<kScan1Threads>(lane == 63 ? carry : 0, smem, &tot);
  const bool ovf = capacity >= 0 && tot > capacity;
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int64_t i = (int64_t)base + 64 * q;
    if (i < n) a[i] = ovf ? 0 : (int32_t)(off + v[q]);
  }
  if (threadIdx.x == 0) {
    a[n] = ovf ? 0 : (int32_t)tot;
    if (capacity >= 0) {
      st->last_n_edges = tot;
      st->overflow = ovf;
      if (ovf) dev_fail(st, SN_ERR_CAPACITY, tot);
    }
  }
}

hipError_t launch_exclusive_scan(int32_t* a, int64_t n, int32_t* blocks_i32, DevStatus* st,
                                 int64_t capacity, const int64_t* gate, int64_t gate_val,
                                 hipStream_t s) {
  if (n <= kScan1Max) {
    const int64_t q = (n + kScan1Threads - 1) / kScan1Threads;   // loads per lane needed
    auto one = [&](auto kern) {
      hipLaunchKernelGGL(kern, dim3(1), dim3(kScan1Threads), 0, s, a, n, st, capacity, gate,
                         gate_val);
      return hipGetLastError();
    };
    if (q <= 4) return one(k_scan_single<4>);
    if (q <= 8) return one(k_scan_single<8>);
    if (q <= 16) return one(k_scan_single<16>);
    return one(k_scan_single<32>);
  }
  int64_t* blocks = reinterpret_cast<int64_t*>(blocks_i32);
  const int64_t nblk = (n + kScanChunk - 1) / kScanChunk;
  hipLaunchKernelGGL(k_scan_local, dim3((unsigned)nblk), dim3(kThreads), 0, s, a, n, blocks, gate,
                     gate_val);
  hipLaunchKernelGGL(k_scan_top, dim3(1), dim3(kThreads), 0, s, blocks, nblk, st, capacity, gate,
                     gate_val);
  hipLaunchKernelGGL(k_scan_add, dim3((unsigned)nblk), dim3(kThreads), 0, s, a, n, blocks, nblk,
                     capacity, gate, gate_val);
  return hipGetLastError();
}

// ------------------------------------------------------------------ all pairs per replica
// One wave per receiver: the lanes test 64 senders of the same replica at a
// time and a ballot compacts the hits in sender order, so each row is written
// sorted, with contiguous stores, and small replicas still give one wave per
// atom of the whole batch.
template <bool FILL>
__global__ __launch_bounds__(kThreads) void k_nbr_allpairs(const float* __restrict__ pos, int N,
                                                           int64_t n_tot, int periodic, double L,
                                                           double half, double r2,
                                                           int32_t* rowptr, int32_t* col,
                                                           DevStatus* st,
                                                           const int64_t* gate, int64_t gate_val) {
  SN_GATE
  if (FILL && st->overflow) return;
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (r >= n_tot) return;
  const int il = (int)(r % N);
  const int64_t base = r - il;
  const float xi = pos[3 * r + 0], yi = pos[3 * r + 1], zi = pos[3 * r + 2];
  if (!FILL && lane == 0) check_position(st, r, xi, yi, zi);
  const uint64_t below = (1ull << lane) - 1ull;
  int64_t out = FILL ? (int64_t)rowptr[r] : 0;
  int cnt = 0;
  for (int j0 = 0; j0 < N; j0 += 64) {
    const int j = j0 + lane;
    bool in = false;
    if (j < N && j != il) {
      const float* pj = pos + 3 * (base + j);
      in = pair_in(xi, yi, zi, pj[0], pj[1], pj[2], periodic, L, half, r2);
    }
    const uint64_t m = __ballot(in);
    if (FILL) {
      if (in) col[out + __popcll(m & below)] = (int32_t)(base + j);
      out += __popcll(m);
    } else {
      cnt += __popcll(m);
    }
  }
  if (!FILL && lane == 0) rowptr[r] = cnt;
}

// ------------------------------------------------------------------ cell list (one periodic cube)
__global__ __launch_bounds__(kThreads) void k_fill_i32(int32_t* p, int64_t n, int32_t v,
                                                       const int64_t* gate, int64_t gate_val) {
  SN_GATE
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kThreads)
    p[i] = v;
}

__device__ __forceinline__ int cell_coord(float x, float inv_cell, int nc) {
  int c = (int)(x * inv_cell);
  return c < 0 ? 0 : (c >= nc ? nc - 1 : c);
}

// Cell grid of an open system, found on the device (k_open_grid): cells
// per axis and, per axis, the lowest coordinate and cells per unit length.
// The cell-list kernels take either this grid (OPEN) or one periodic cube
// (nc cells per axis of 1 / inv_cell each, from the origin).
struct CellGrid {
  int nx, ny, nz;
  float lo[3], inv[3];
  __device__ __forceinline__ int cell_of(float x, float y, float z) const {
    const int cx = cell_coord(x - lo[0], inv[0], nx);
    const int cy = cell_coord(y - lo[1], inv[1], ny);
    const int cz = cell_coord(z - lo[2], inv[2], nz);
    return (cz * ny + cy) * nx + cx;
  }
};
static_assert(sizeof(CellGrid) <= 64, "the workspace keeps 64 bytes for the grid");
__device__ __forceinline__ CellGrid cube_grid(float inv_cell, int nc) {
  CellGrid g;
  g.nx = g.ny = g.nz = nc;
  for (int a = 0; a < 3; ++a) {
    g.lo[a] = 0.f;
    g.inv[a] = inv_cell;
  }
  return g;
}

// The bounding box of an open system (one work-group; min and max are
// independent of order) and the grid over it: per axis the largest number of
// cells, at most kCellsPerAxisMax, whose edge is at least r_list (one cell
// where the extent is below r_list).
__global__ __launch_bounds__(1024) void k_open_grid(const float* __restrict__ pos, int N,
                                                    double r_list, CellGrid* grid,
                                                    const int64_t* gate, int64_t gate_val) {
  SN_GATE
  __shared__ float smin[3][16], smax[3][16];
  float lo[3] = {INFINITY, INFINITY, INFINITY}, hi[3] = {-INFINITY, -INFINITY, -INFINITY};
  for (int i = threadIdx.x; i < N; i += 1024)
    for (int a = 0; a < 3; ++a) {
      const float v = pos[3 * i + a];
      lo[a] = fminf(lo[a], v);
      hi[a] = fmaxf(hi[a], v);
    }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int a = 0; a < 3; ++a) {
    for (int o = 32; o > 0; o >>= 1) {
      lo[a] = fminf(lo[a], __shfl_xor(lo[a], o, 64));
      hi[a] = fmaxf(hi[a], __shfl_xor(hi[a], o, 64));
    }
    if (lane == 0) {
      smin[a][wave] = lo[a];
      smax[a][wave] = hi[a];
    }
  }
  __syncthreads();
  if (threadIdx.x != 0) return;
  CellGrid g;
  int n[3];
  for (int a = 0; a < 3; ++a) {
    float l = smin[a][0], h = smax[a][0];
    for (int w = 1; w < 16; ++w) {
      l = fminf(l, smin[a][w]);
      h = fmaxf(h, smax[a][w]);
    }
    const double ext = (double)h - (double)l;
    double c = ext / (r_list * (1.0 + 1e-5));
    n[a] = (c >= 1.0 && ext < INFINITY) ? (c >= kCellsPerAxisMax ? kCellsPerAxisMax : (int)c) : 1;
    g.lo[a] = (ext < INFINITY) ? l : 0.f;
    g.inv[a] = n[a] > 1 ? (float)((double)n[a] / ext) : 0.f;
  }
  g.nx = n[0];
  g.ny = n[1];
  g.nz = n[2];
  *grid = g;
}

template <bool OPEN>
__global__ __launch_bounds__(kThreads) void k_cell_assign(const float* __restrict__ pos, int N,
                                                          float inv_cell, int nc,
                                                          const CellGrid* open_grid,
                                                          int32_t* atom_cell,
                                                          int32_t* cell_count, DevStatus* st,
                                                          const int64_t* gate, int64_t gate_val) {
  SN_GATE
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i >= N) return;
  check_position(st, i, pos[3 * i + 0], pos[3 * i + 1], pos[3 * i + 2]);
  const CellGrid g = OPEN ? *open_grid : cube_grid(inv_cell, nc);
  const int c = g.cell_of(pos[3 * i + 0], pos[3 * i + 1], pos[3 * i + 2]);
  atom_cell[i] = c;
  atomicAdd(&cell_count[c], 1);
}

__global__ __launch_bounds__(kThreads) void k_cell_scatter(int N, const int32_t* atom_cell,
                                                           const int32_t* cell_start,
                                                           int32_t* cell_cursor, int32_t* cell_atoms,
                                                           const int64_t* gate, int64_t gate_val) {
  SN_GATE
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i >= N) return;
  const int c = atom_cell[i];
  const int slot = atomicAdd(&cell_cursor[c], 1);
  cell_atoms[cell_start[c] + slot] = i;
}

// One wave per receiver i. The members of the 27 cells around i's cell form
// one candidate list (cell order, then slot order); lanes take 64 candidates
// at a time, each finding its cell by a binary search over the cells'
// offsets, so the loads of a round are independent. Hits are compacted with a
// ballot; k_sort_rows orders each row afterwards. A periodic cube wraps the
// neighbouring cells around (27 distinct cells, nc >= 3); an open grid leaves
// out those past its faces.
template <bool FILL, bool OPEN>
__global__ __launch_bounds__(kThreads) void k_nbr_cells(const float* __restrict__ pos, int N,
                                                        int n_per, int nc,
                                                        const CellGrid* open_grid,
                                                        double L, double half, double r2,
                                                        const int32_t* atom_cell,
                                                        const int32_t* cell_start,
                                                        const int32_t* cell_atoms, int32_t* rowptr,
                                                        int32_t* col, const DevStatus* st,
                                                        const int64_t* gate, int64_t gate_val) {
  SN_GATE
  if (FILL && st->overflow) return;
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (i >= N) return;
  const float xi = pos[3 * i + 0], yi = pos[3 * i + 1], zi = pos[3 * i + 2];
  // the receiver's replica: atoms [rlo, rlo + n_per) (cells hold every replica's atoms)
  const int rlo = i - i % n_per;
  const int c = atom_cell[i];
  const int nx = OPEN ? open_grid->nx : nc, ny = OPEN ? open_grid->ny : nc,
            nz = OPEN ? open_grid->nz : nc;
  const int cx = c % nx, cy = (c / nx) % ny, cz = c / (nx * ny);
  // lanes 0..26: start and size of one neighbouring cell
  int cs = 0, cn = 0;
  if (lane < 27) {
    const int dz = lane / 9 - 1, dy = (lane / 3) % 3 - 1, dx = lane % 3 - 1;
    int ax = cx + dx, ay = cy + dy, az = cz + dz;
    bool ok = true;
    if (OPEN) {
      ok = ax >= 0 && ax < nx && ay >= 0 && ay < ny && az >= 0 && az < nz;
    } else {
      ax = (ax + nx) % nx;
      ay = (ay + ny) % ny;
      az = (az + nz) % nz;
    }
    if (ok) {
      const int cc = (az * ny + ay) * nx + ax;
      cs = cell_start[cc];
      cn = cell_start[cc + 1] - cs;
    }
  }
  int incl = cn;
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  const int excl = incl - cn;
  const int total = __shfl(incl, 26, 64);
  int64_t out = FILL ? rowptr[i] : 0;
  int cnt = 0;
  for (int f0 = 0; f0 < total; f0 += 64) {
    const int f = f0 + lane;
    // the last cell whose offset is <= f (empty cells share the next cell's offset)
    int lo = 0, hi = 26;
#pragma unroll
    for (int step = 0; step < 5; ++step) {
      const int mid = (lo + hi + 1) >> 1;
      if (__shfl(excl, mid, 64) <= f) lo = mid;
      else hi = mid - 1;
    }
    const int k = __shfl(cs, lo, 64) + (f - __shfl(excl, lo, 64));
    bool in = false;
    int j = 0;
    if (f < total) {
      j = cell_atoms[k];
      in = j != i && (unsigned)(j - rlo) < (unsigned)n_per &&
           pair_in(xi, yi, zi, pos[3 * j], pos[3 * j + 1], pos[3 * j + 2], OPEN ? 0 : 1, L, half,
                   r2);
    }
    const uint64_t m = __ballot(in);
    if (FILL && in) col[out + __popcll(m & ((1ull << lane) - 1))] = j;
    const int nh = __popcll(m);
    out += nh;
    cnt += nh;
  }
  if (!FILL && lane == 0) rowptr[i] = cnt;
}

// Rank sort of each row (distinct values), one wave per row, staged in LDS.
__global__ __launch_bounds__(kThreads) void k_sort_rows(const int32_t* rowptr, int32_t* col, int N,
                                                        DevStatus* st, const int64_t* gate,
                                                        int64_t gate_val) {
  SN_GATE
  if (st->overflow) return;
  __shared__ int32_t buf[kThreads / 64][kSortRowMax];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.x * (kThreads / 64) + wave;
  int s = 0, n = 0;
  if (row < N) {
    s = rowptr[row];
    n = rowptr[row + 1] - s;
    if (n > kSortRowMax) {
      if (lane == 0) dev_fail(st, SN_ERR_UNSUPPORTED, row);
      n = 0;
    }
  }
  for (int e = lane; e < n; e += 64) buf[wave][e] = col[s + e];
  __syncthreads();
  for (int e = lane; e < n; e += 64) {
    const int v = buf[wave][e];
    int rank = 0;
    for (int k = 0; k < n; ++k) rank += buf[wave][k] < v;
    col[s + rank] = v;
  }
}

// ------------------------------------------------------------------ active list
// The rows of a list restricted to the pairs that pass the membership test at
// a smaller radius, in the same order. Each row is taken by LPR lanes (64 /
// LPR rows per wave: rows are short) that test LPR listed senders at a time;
// a ballot compacts the kept ones within the row's lane group. The count pass
// (FILL false) writes row lengths into out_rowptr, the fill pass the senders
// at the scanned offsets.
template <bool FILL, int LPR>
__global__ __launch_bounds__(kThreads) void k_active(const float* __restrict__ pos, int64_t n_tot,
                                                     int periodic, double L, double half,
                                                     double r2, const int32_t* __restrict__ rowptr,
                                                     const int32_t* __restrict__ col,
                                                     int32_t* out_rowptr, int32_t* out_col) {
  const int lane = threadIdx.x & 63, sub = lane % LPR, grp = lane / LPR;
  const int64_t r = ((int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)) * (64 / LPR) + grp;
  const bool row_ok = r < n_tot;
  const int b = row_ok ? rowptr[r] : 0, e = row_ok ? rowptr[r + 1] : 0;
  float xi = 0.f, yi = 0.f, zi = 0.f;
  if (row_ok) {
    xi = pos[3 * r + 0];
    yi = pos[3 * r + 1];
    zi = pos[3 * r + 2];
  }
  const uint64_t gmask = (LPR == 64 ? ~0ull : ((1ull << LPR) - 1ull)) << (grp * LPR);
  const uint64_t below = ((1ull << lane) - 1ull) & gmask;
  int64_t out = (FILL && row_ok) ? (int64_t)out_rowptr[r] : 0;
  // every lane group of the wave loops as long as its longest row needs
  int len = e - b;
  for (int o = LPR; o < 64; o <<= 1) len = max(len, __shfl_xor(len, o, 64));
  for (int k0 = 0; k0 < len; k0 += LPR) {
    const int k = b + k0 + sub;
    bool in = false;
    int j = 0;
    if (k < e) {
      j = col[k];
      const float* pj = pos + 3 * (int64_t)j;
      in = pair_in(xi, yi, zi, pj[0], pj[1], pj[2], periodic, L, half, r2);
    }
    const uint64_t m = __ballot(in);
    if (FILL && in) out_col[out + __popcll(m & below)] = j;
    out += __popcll(m & gmask);
  }
  if (!FILL && row_ok && sub == 0) out_rowptr[r] = (int32_t)out;
}

hipError_t launch_active_list(const NbrGeom& g, const float* pos, const int32_t* rowptr,
                              const int32_t* col, double r2, int32_t* out_rowptr,
                              int32_t* out_col, char* ws, const WsLayout& L, hipStream_t s) {
  constexpr int LPR = 16;
  DevStatus* st = reinterpret_cast<DevStatus*>(ws + L.status);
  int32_t* scan_blocks = reinterpret_cast<int32_t*>(ws + L.scan_blocks);
  const int64_t n_tot = (int64_t)g.n_rep * g.n_per;
  const int64_t rows_per_block = (kThreads / 64) * (64 / LPR);
  const dim3 grid((unsigned)((n_tot + rows_per_block - 1) / rows_per_block));
  hipLaunchKernelGGL((k_active<false, LPR>), grid, dim3(kThreads), 0, s, pos, n_tot, g.periodic,
                     g.L, g.half, r2, rowptr, col, out_rowptr, out_col);
  hipError_t e = launch_exclusive_scan(out_rowptr, n_tot, scan_blocks, st, -1, nullptr, 0, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_active<true, LPR>), grid, dim3(kThreads), 0, s, pos, n_tot, g.periodic,
                     g.L, g.half, r2, rowptr, col, out_rowptr, out_col);
  return hipGetLastError();
}

static unsigned blocks_for(int64_t n) { return (unsigned)((n + kThreads - 1) / kThreads); }

hipError_t launch_build_neighbors(const NbrGeom& g, const float* pos, int32_t* rowptr, int32_t* col,
                                  int64_t edge_capacity, char* ws, const WsLayout& L,
                                  const int64_t* gate, int64_t gate_val, hipStream_t s) {
  DevStatus* st = reinterpret_cast<DevStatus*>(ws + L.status);
  int32_t* scan_blocks = reinterpret_cast<int32_t*>(ws + L.scan_blocks);
  const int64_t n_tot = (int64_t)g.n_rep * g.n_per;
  hipError_t e;
  if (g.cells_per_axis == 0) {
    const dim3 grid((unsigned)((n_tot + kThreads / 64 - 1) / (kThreads / 64)));
    hipLaunchKernelGGL(k_nbr_allpairs<false>, grid, dim3(kThreads), 0, s, pos, g.n_per, n_tot,
                       g.periodic, g.L, g.half, g.r2, rowptr, col, st, gate, gate_val);
    if ((e = launch_exclusive_scan(rowptr, n_tot, scan_blocks, st, edge_capacity, gate, gate_val,
                                   s)) != hipSuccess)
      return e;
    hipLaunchKernelGGL(k_nbr_allpairs<true>, grid, dim3(kThreads), 0, s, pos, g.n_per, n_tot,
                       g.periodic, g.L, g.half, g.r2, rowptr, col, st, gate, gate_val);
    return hipGetLastError();
  }
  // a periodic cube of nc^3 cells, or an open grid of up to kCellsPerAxisMax^3
  // cells whose sizes the device sets (cells past its own count stay empty)
  const bool open = g.cells_per_axis < 0;
  const int nc = open ? 0 : g.cells_per_axis;
  const int64_t ncell = open ? (int64_t)kCellsPerAxisMax * kCellsPerAxisMax * kCellsPerAxisMax
                             : (int64_t)nc * nc * nc;
  CellGrid* grid = reinterpret_cast<CellGrid*>(ws + L.cell_grid);
  int32_t* cstart = reinterpret_cast<int32_t*>(ws + L.cell_count);   // counts, then starts
  int32_t* ccur = reinterpret_cast<int32_t*>(ws + L.cell_start);     // scatter cursors
  int32_t* catoms = reinterpret_cast<int32_t*>(ws + L.cell_atoms);
  int32_t* acell = reinterpret_cast<int32_t*>(ws + L.atom_cell);
  const int N = g.n_rep * g.n_per;   // every replica's atoms share the cells
  hipLaunchKernelGGL(k_fill_i32, dim3(blocks_for(ncell + 1)), dim3(kThreads), 0, s, cstart,
                     ncell + 1, 0, gate, gate_val);
  hipLaunchKernelGGL(k_fill_i32, dim3(blocks_for(ncell)), dim3(kThreads), 0, s, ccur, ncell, 0,
                     gate, gate_val);
  if (open) {
    hipLaunchKernelGGL(k_open_grid, dim3(1), dim3(1024), 0, s, pos, N, std::sqrt(g.r2), grid, gate,
                       gate_val);
    hipLaunchKernelGGL(k_cell_assign<true>, dim3(blocks_for(N)), dim3(kThreads), 0, s, pos, N,
                       0.f, 0, grid, acell, cstart, st, gate, gate_val);
  } else {
    hipLaunchKernelGGL(k_cell_assign<false>, dim3(blocks_for(N)), dim3(kThreads), 0, s, pos, N,
                       g.inv_cell, nc, grid, acell, cstart, st, gate, gate_val);
  }
  if ((e = launch_exclusive_scan(cstart, ncell, scan_blocks, st, -1, gate, gate_val, s)) !=
      hipSuccess)
    return e;
  hipLaunchKernelGGL(k_cell_scatter, dim3(blocks_for(N)), dim3(kThreads), 0, s, N, acell, cstart,
                     ccur, catoms, gate, gate_val);
  const dim3 wave_grid((unsigned)((N + kThreads / 64 - 1) / (kThreads / 64)));
  if (open)
    hipLaunchKernelGGL((k_nbr_cells<false, true>), wave_grid, dim3(kThreads), 0, s, pos, N,
                       g.n_per, nc, grid, g.L, g.half, g.r2, acell, cstart, catoms, rowptr, col, st, gate,
                       gate_val);
  else
    hipLaunchKernelGGL((k_nbr_cells<false, false>), wave_grid, dim3(kThreads), 0, s, pos, N,
                       g.n_per, nc, grid, g.L, g.half, g.r2, acell, cstart, catoms, rowptr, col, st, gate,
                       gate_val);
  if ((e = launch_exclusive_scan(rowptr, N, scan_blocks, st, edge_capacity, gate, gate_val, s)) !=
      hipSuccess)
    return e;
  if (open)
    hipLaunchKernelGGL((k_nbr_cells<true, true>), wave_grid, dim3(kThreads), 0, s, pos, N,
                       g.n_per, nc, grid, g.L, g.half, g.r2, acell, cstart, catoms, rowptr, col, st, gate,
                       gate_val);
  else
    hipLaunchKernelGGL((k_nbr_cells<true, false>), wave_grid, dim3(kThreads), 0, s, pos, N,
                       g.n_per, nc, grid, g.L, g.half, g.r2, acell, cstart, catoms, rowptr, col, st, gate,
                       gate_val);
  hipLaunchKernelGGL(k_sort_rows, dim3((unsigned)((N + 3) / 4)), dim3(kThreads), 0, s, rowptr, col,
                     N, st, gate, gate_val);
  return hipGetLastError();
}

} // namespace sn
