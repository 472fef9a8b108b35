// The local KNN decoder's gather on gfx950: the AVS-Conv operator of the
// MSVS-VAE page (kwkr.cn), section 1.1. A query takes its K nearest supports
// (Euclidean distance), turns each neighbour's offset into per-channel dynamic
// weights through an MLP, and fuses the neighbours' features by a weighted sum
// plus a mean-pool residual:
//   h = (1/K) sum_j (B GELU(A delta_j + a)) * f_j + (1/K) sum_j f_j,  delta_j = p_j - x.
// The head (y = h + W2 GELU(W1 h), SDF) runs in k_decode.hip's epilogue code.
//
// Stages:
//   grid   the supports are bucketed into a LOCAL_G^3 grid of cells over
//          [-1, 1]^3 (count, scan, scatter); each bucket entry carries the
//          support's position and index;
//   knn    the queries are bucketed the same way, for a cell-ordered
//          processing order; one thread per query walks shells of cells around
//          its own (Chebyshev rings of growing radius) through per-row
//          occupancy words in LDS, skips cells whose box lies beyond the current
//          K-th distance, keeps the K smallest (distance, index) pairs, and stops
//          once every cell outside the scanned block lies farther than that;
//   fuse   one wave per pair of queries (2 x 16 neighbours = one 32-row MFMA
//          block): the offset MLP's hidden units in registers (exact-erf GELU),
//          the dynamic weights w = G B^T on bf16 MFMA (hidden width 32 = two
//          k-steps), the neighbours' feature rows staged in the wave's LDS slice,
//          and the sum over the 16 rows of each query in registers.
#include "vdm_device.hpp"

namespace vdm {

// ------------------------------------------------------------------ support grid

constexpr float LOCAL_CELLS_PER_UNIT = LOCAL_G / 2.0f;  // cell edge 2 / LOCAL_G (a power of two)
constexpr int LOCAL_NC = LOCAL_G * LOCAL_G * LOCAL_G;
static_assert(LOCAL_G == 32, "one 32-bit occupancy word per row of cells along z");

// Cell coordinate of c along one axis, clamped into [0, LOCAL_G); NaN goes to 0.
__device__ __forceinline__ int local_cell(float c) {
  float t = (c + 1.f) * LOCAL_CELLS_PER_UNIT;
  t = fminf(fmaxf(t, 0.f), (float)(LOCAL_G - 1));
  return (int)t;
}

__device__ __forceinline__ int local_cell_id(int i, int j, int k) { return (i * LOCAL_G + j) * LOCAL_G + k; }

__device__ __forceinline__ int local_cell_of(const float* p) {
  return local_cell_id(local_cell(p[0]), local_cell(p[1]), local_cell(p[2]));
}

// counts[cell] += 1 for each point; cell_of[point] = its cell
__global__ void local_count_kernel(const float* __restrict__ xyz, int64_t n, int32_t* counts, int32_t* cell_of) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= n) return;
  const int c = local_cell_of(xyz + 3 * j);
  cell_of[j] = c;
  atomicAdd(&counts[c], 1);
}

// Exclusive prefix sum of the LOCAL_NC counts into starts[0 .. LOCAL_NC] by one
// workgroup of 1024 threads, 32 consecutive cells per thread; with occ != null
// also the occupancy words occ[i * LOCAL_G + j] (bit k: cell (i, j, k) holds a point).
__global__ __launch_bounds__(1024) void local_scan_kernel(const int32_t* __restrict__ counts, int32_t* starts,
                                                          uint32_t* occ) {
  constexpr int PER = LOCAL_NC / 1024;
  static_assert(PER == LOCAL_G, "a thread's run is one row of cells");
  __shared__ int32_t part[1024];
  const int t = threadIdx.x;
  int32_t sum = 0;
  uint32_t bits = 0;
  for (int i = 0; i < PER; ++i) {
    const int32_t c = counts[t * PER + i];
    sum += c;
    bits |= (c > 0 ? 1u : 0u) << i;
  }
  if (occ) occ[t] = bits;
  part[t] = sum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {  // Hillis-Steele inclusive scan of the run sums
    const int32_t v = t >= off ? part[t - off] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int32_t run = part[t] - sum;  // exclusive start of this thread's run
  for (int i = 0; i < PER; ++i) {
    starts[t * PER + i] = run;
    run += counts[t * PER + i];
  }
  if (t == 1023) starts[LOCAL_NC] = run;
}

// Points in cell order: spos (x, y, z, index bits) for supports, or the index
// alone (order) for queries.
__global__ void local_scatter_kernel(const float* __restrict__ xyz, int64_t n, const int32_t* __restrict__ cell_of,
                                     const int32_t* __restrict__ starts, int32_t* fill, float4* spos,
                                     int32_t* order) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= n) return;
  const int c = cell_of[j];
  const int at = starts[c] + atomicAdd(&fill[c], 1);
  if (!VDM_BOUND(at >= 0 && at < n, BC_LOCAL_SCATTER)) return;
  if (spos) spos[at] = make_float4(xyz[3 * j], xyz[3 * j + 1], xyz[3 * j + 2], __int_as_float((int)j));
  if (order) order[at] = (int32_t)j;
}

hipError_t launch_local_grid(const float* xyz, int64_t n, int32_t* counts, int32_t* starts, int32_t* fill,
                             int32_t* cell_of, float4* spos, int32_t* order, uint32_t* occ, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const unsigned g = (unsigned)((n + 255) / 256);
  hipLaunchKernelGGL(local_count_kernel, dim3(g), dim3(256), 0, s, xyz, n, counts, cell_of);
  hipLaunchKernelGGL(local_scan_kernel, dim3(1), dim3(1024), 0, s, counts, starts, occ);
  hipLaunchKernelGGL(local_scatter_kernel, dim3(g), dim3(256), 0, s, xyz, n, cell_of, starts, fill, spos, order);
  return hipGetLastError();
}

// ------------------------------------------------------------------ K nearest supports

// float32 squared distance in the stated order, with no fused multiply-add:
// fl(fl(fl(dx dx) + fl(dy dy)) + fl(dz dz)), dx = fl(p_x - x_x).
__device__ __forceinline__ float sq_dist(float px, float py, float pz, float x, float y, float z) {
#pragma clang fp contract(off)
  const float dx = px - x, dy = py - y, dz = pz - z;
  const float sx = dx * dx, sy = dy * dy, sz = dz * dz;
  return (sx + sy) + sz;
}

// (d, j) before (e, k): smaller distance, then smaller index
__device__ __forceinline__ bool knn_less(float d, int j, float e, int k) { return d < e || (d == e && j < k); }

// true when every point at least r from the query lies strictly beyond the K-th
// squared distance kd (margins for the rounding of points' cells and of distances)
__device__ __forceinline__ bool beyond_kth(float r, float kd) {
  const float rr = r - 1e-6f;
  return rr > 0.f && rr * rr * (1.f - 1e-5f) > kd;
}

constexpr int KNN_THREADS = 256;

// One thread per query, the queries taken in cell order (order[]) so that the
// lanes of a wave walk nearby shells. The shell of Chebyshev radius s around the
// query's cell is enumerated row by row (i, j); a row's occupied cells come from
// its occupancy word (LDS), and a cell whose box lies beyond the current K-th
// distance is skipped (a border cell's box is open towards the outside, where
// clamped points may lie).
__global__ __launch_bounds__(KNN_THREADS) void local_knn_kernel(const float* __restrict__ xyz, int64_t N,
                                                                const int32_t* __restrict__ order,
                                                                const int32_t* __restrict__ starts,
                                                                const uint32_t* __restrict__ occ_g,
                                                                const float4* __restrict__ spos,
                                                                int32_t* __restrict__ nbr) {
  __shared__ uint32_t occ[LOCAL_G * LOCAL_G];
  for (int i = threadIdx.x; i < LOCAL_G * LOCAL_G; i += KNN_THREADS) occ[i] = occ_g[i];
  __syncthreads();
  const int64_t t = (int64_t)blockIdx.x * KNN_THREADS + threadIdx.x;
  if (t >= N) return;
  const int64_t q = order[t];
  if (!VDM_BOUND(q >= 0 && q < N, BC_LOCAL_QUERY)) return;
  [[maybe_unused]] const int mtot = VDM_DEBUG ? starts[LOCAL_NC] : 0;  // the support count (bounds-checked builds)
  const float x = xyz[3 * q], y = xyz[3 * q + 1], z = xyz[3 * q + 2];
  const int c[3] = {local_cell(x), local_cell(y), local_cell(z)};
  const float xv[3] = {x, y, z};
  constexpr float H = 2.0f / LOCAL_G;
  float bd[LOCAL_K];
  int bj[LOCAL_K];
#pragma unroll
  for (int i = 0; i < LOCAL_K; ++i) {
    bd[i] = __builtin_inff();
    bj[i] = 0x7fffffff;
  }
  // squared distance from the query to the box of cell index ci along axis a
  auto axis_gap = [&](int a, int ci) -> float {
    const float lo = ci == 0 ? -__builtin_inff() : -1.f + (float)ci * H;
    const float hi = ci == LOCAL_G - 1 ? __builtin_inff() : -1.f + (float)(ci + 1) * H;
    return fmaxf(fmaxf(lo - xv[a], xv[a] - hi), 0.f);
  };
  auto take = [&](const float4 p) {
    const float d = sq_dist(p.x, p.y, p.z, x, y, z);
    const int j = __float_as_int(p.w);
    if (knn_less(d, j, bd[LOCAL_K - 1], bj[LOCAL_K - 1])) {
      bd[LOCAL_K - 1] = d;
      bj[LOCAL_K - 1] = j;
#pragma unroll
      for (int i = LOCAL_K - 1; i > 0; --i) {
        if (knn_less(bd[i], bj[i], bd[i - 1], bj[i - 1])) {
          const float td = bd[i];
          bd[i] = bd[i - 1];
          bd[i - 1] = td;
          const int tj = bj[i];
          bj[i] = bj[i - 1];
          bj[i - 1] = tj;
        }
      }
    }
  };
  // the supports spos[lo .. hi), four loads in flight at a time
  auto visit = [&](int lo, int hi) {
    if (!VDM_BOUND(lo >= 0 && lo <= hi && (!VDM_DEBUG || hi <= mtot), BC_LOCAL_RANGE)) return;
    int u = lo;
    for (; u + 4 <= hi; u += 4) {
      const float4 p0 = spos[u], p1 = spos[u + 1], p2 = spos[u + 2], p3 = spos[u + 3];
      take(p0);
      take(p1);
      take(p2);
      take(p3);
    }
    for (; u < hi; ++u) take(spos[u]);
  };
  for (int s = 0; s <= LOCAL_G; ++s) {
    const int k0 = max(c[2] - s, 0), k1 = min(c[2] + s, LOCAL_G - 1);
    const uint32_t span = (k1 - k0 == 31 ? 0xffffffffu : ((1u << (k1 - k0 + 1)) - 1u)) << k0;
    uint32_t ends = 0;
    if (c[2] - s >= 0) ends |= 1u << (c[2] - s);
    if (c[2] + s < LOCAL_G) ends |= 1u << (c[2] + s);
    for (int di = -s; di <= s; ++di) {
      const int ci = c[0] + di;
      if (ci < 0 || ci >= LOCAL_G) continue;
      const bool fi = di == -s || di == s;
      const float gi = axis_gap(0, ci);
      for (int dj = -s; dj <= s; ++dj) {
        const int cj = c[1] + dj;
        if (cj < 0 || cj >= LOCAL_G) continue;
        const bool face = fi || dj == -s || dj == s;
        uint32_t m = occ[ci * LOCAL_G + cj] & (face ? span : ends);
        if (!m) continue;
        if (bj[LOCAL_K - 1] != 0x7fffffff) {
          // cells along z whose box can hold a point within the K-th distance
          // (inflated for rounding): the interval [z - gz, z + gz]
          const float gj = axis_gap(1, cj);
          const float R = sqrtf(bd[LOCAL_K - 1]) * (1.f + 1e-5f) + 2e-6f;
          const float rem = R * R - (gi * gi + gj * gj);
          if (rem < 0.f) continue;
          const float gz = sqrtf(rem) + 1e-6f;
          const int ka = local_cell(z - gz), kb = local_cell(z + gz);
          m &= (kb - ka == 31 ? 0xffffffffu : ((1u << (kb - ka + 1)) - 1u)) << ka;
          if (!m) continue;
        }
        const int row = (ci * LOCAL_G + cj) * LOCAL_G;
        if (face) {
          // the occupied cells of the row segment are contiguous in cell order
          const int kf = __builtin_ctz(m), kl = 31 - __builtin_clz(m);
          visit(starts[row + kf], starts[row + kl + 1]);
        } else {
          while (m) {
            const int ck = __builtin_ctz(m);
            m &= m - 1;
            visit(starts[row + ck], starts[row + ck + 1]);
          }
        }
      }
    }
    // every support outside the block of scanned cells lies beyond one of the
    // block's faces that has cells behind it: at least r from the query
    float r = __builtin_inff();
    bool beyond = false;
#pragma unroll
    for (int a = 0; a < 3; ++a) {
      if (c[a] - s > 0) {
        beyond = true;
        r = fminf(r, xv[a] - (-1.f + (float)(c[a] - s) * H));
      }
      if (c[a] + s < LOCAL_G - 1) {
        beyond = true;
        r = fminf(r, (-1.f + (float)(c[a] + s + 1) * H) - xv[a]);
      }
    }
    if (!beyond) break;  // the whole grid has been scanned
    if (bj[LOCAL_K - 1] != 0x7fffffff && beyond_kth(r, bd[LOCAL_K - 1])) break;
  }
#pragma unroll
  for (int i = 0; i < LOCAL_K; ++i) nbr[q * LOCAL_K + i] = bj[i];
}

hipError_t launch_local_knn(const float* xyz, int64_t N, const int32_t* order, const int32_t* starts,
                            const uint32_t* occ, const float4* spos, int32_t* nbr, hipStream_t s) {
  if (N <= 0) return hipSuccess;
  hipLaunchKernelGGL(local_knn_kernel, dim3((unsigned)((N + KNN_THREADS - 1) / KNN_THREADS)), dim3(KNN_THREADS), 0, s,
                     xyz, N, order, starts, occ, spos, nbr);
  return hipGetLastError();
}

// ------------------------------------------------------------------ fusion (AVS-Conv)

constexpr int FUSE_WAVES = 4;
constexpr int FROW = LOCAL_C + 8;  // LDS row of one neighbour's features (bf16, padded)

__global__ __launch_bounds__(64 * FUSE_WAVES) void local_fuse_kernel(LocalFuseArgs A) {
  extern __shared__ __align__(16) char lds[];
  using MM = Mma<bf16>;
  using Frag = MM::frag;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  bf16* Fs = reinterpret_cast<bf16*>(lds) + wave * 32 * FROW;
  const bf16* __restrict__ Bw = reinterpret_cast<const bf16*>(A.B);
  const bf16* __restrict__ feats = reinterpret_cast<const bf16*>(A.feats);
  const int half = lane >> 5, p = lane & 31;

  // B fragments of the 8 channel blocks (B operand: channel = column, hidden = k)
  Frag bf[LOCAL_C / 32][2];
#pragma unroll
  for (int cb = 0; cb < LOCAL_C / 32; ++cb)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      bf[cb][ks] = *reinterpret_cast<const Frag*>(Bw + (32 * cb + p) * LOCAL_HIDDEN + 16 * ks + 8 * half);
  // the offset MLP's first layer, (A row, a) per hidden unit, in LDS after the wave slices
  float4* Aa = reinterpret_cast<float4*>(lds + FUSE_WAVES * 32 * FROW * 2);
  for (int m = threadIdx.x; m < LOCAL_HIDDEN; m += blockDim.x)
    Aa[m] = make_float4(A.A[3 * m], A.A[3 * m + 1], A.A[3 * m + 2], A.a[m]);
  __syncthreads();

  const int64_t npairs = (A.N + 1) / 2;
  for (int64_t it = (int64_t)blockIdx.x * FUSE_WAVES + wave; it < npairs; it += (int64_t)gridDim.x * FUSE_WAVES) {
    // pair row p: query 2 it + p / 16 (the last query repeats for an odd N), neighbour p % 16
    const int64_t q = min(2 * it + (p >> 4), A.N - 1);
    int j = A.nbr[q * LOCAL_K + (p & 15)];
    j = j < 0 ? 0 : (j >= A.M ? A.M - 1 : j);
    // (every lane has finished reading the previous pair's rows)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // the 32 neighbours' feature rows into this wave's LDS slice: row 2 i + half,
    // 16-byte chunk p of the row
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int tok = __shfl(j, 2 * i + half);
      *reinterpret_cast<uint4*>(Fs + (2 * i + half) * FROW + 8 * p) =
          *reinterpret_cast<const uint4*>(feats + (int64_t)tok * LOCAL_C + 8 * p);
    }
    // the offset MLP's hidden units m = 16 ks + 8 half + v of this lane's pair,
    // as bf16 A fragments
    const float dx = __fsub_rn(A.sup_xyz[3 * j], A.xyz[3 * q]);
    const float dy = __fsub_rn(A.sup_xyz[3 * j + 1], A.xyz[3 * q + 1]);
    const float dz = __fsub_rn(A.sup_xyz[3 * j + 2], A.xyz[3 * q + 2]);
    Frag g[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      float u[8];
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const float4 w = Aa[16 * ks + 8 * half + v];
        u[v] = gelu(__builtin_fmaf(w.z, dz, __builtin_fmaf(w.y, dy, __builtin_fmaf(w.x, dx, w.w))));
      }
      g[ks] = cvt8(u);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // per channel block: w = G B^T (rows: the 32 pairs), then sum over each
    // query's 16 rows of (w + 1) f / K (1/K = 1/16: exact)
    const int64_t qs = 2 * it + half;  // the query this lane stores
    bf16* hout = reinterpret_cast<bf16*>(A.h) + qs * LOCAL_C;
#pragma unroll
    for (int cb = 0; cb < LOCAL_C / 32; ++cb) {
      f32x16 w = MM::mma(g[0], bf[cb][0], zero16());
      w = MM::mma(g[1], bf[cb][1], w);
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float f = (float)Fs[crow(r, lane) * FROW + 32 * cb + p];
        const float t = __builtin_fmaf(w[r], 1.f / LOCAL_K, 1.f / LOCAL_K) * f;
        if (r < 8)
          s0 += t;
        else
          s1 += t;
      }
      s0 += __shfl_xor(s0, 32);
      s1 += __shfl_xor(s1, 32);
      if (qs < A.N) hout[32 * cb + p] = (bf16)(half ? s1 : s0);
    }
  }
}

hipError_t launch_local_fuse(const LocalFuseArgs& a, hipStream_t s) {
  if (a.N <= 0) return hipSuccess;
  constexpr int lds = FUSE_WAVES * 32 * FROW * 2 + LOCAL_HIDDEN * 16;
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&local_fuse_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    attr = true;
  }
  int per_cu = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, local_fuse_kernel, 64 * FUSE_WAVES, lds);
  if (e != hipSuccess) return e;
  if (per_cu < 1) per_cu = 1;
  int64_t grid = (int64_t)dev_info().cus * per_cu;
  const int64_t need = ((a.N + 1) / 2 + FUSE_WAVES - 1) / FUSE_WAVES;
  if (need < grid) grid = need;
  hipLaunchKernelGGL(local_fuse_kernel, dim3((unsigned)grid), dim3(64 * FUSE_WAVES), lds, s, a);
  return hipGetLastError();
}

VDM_DEBUG_READER(debug_take_local)

}  // namespace vdm
