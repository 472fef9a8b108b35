// Surface extraction from the decoded SDF volume: marching cubes at SDF = 0.
//
// Surface extraction is the stage after VAE decoding in a vecset diffusion
// pipeline (techwalker article on FlashVDM, part 1, the four stages); the pages
// leave the algorithm open, and this is the plainest reading for an SDF sampled on
// a grid. Definition:
//   - a grid point is inside when its value is < 0 (0 and NaN are outside);
//   - every grid edge whose end points differ in that test carries one vertex at
//     the zero of the linear interpolant, t = v0 / (v0 - v1) from the lower end;
//     vertices are numbered by ascending edge id a * P^3 + point index (P = R + 1);
//   - a cell's surface is built face by face: two crossing edges on a face are
//     joined by one segment, four (inside corners on a diagonal) by two segments
//     that each cut off an inside corner; segments are directed so the normal
//     points from the inside corners to the outside ones and chain into loops;
//   - each loop becomes a fan around the vertex of smallest edge id among those
//     that share no cube face with a non-neighbouring loop vertex (no triangle or
//     inner fan edge then lies in a face the next cell also triangulates); loops
//     of a cell in order of their smallest edge id, cells in row-major order.
//
// GPU layout: one bit per grid edge, per axis a bit plane of ceil(P^3 / 64)
// words (bit = point index); a vertex id is the rank of its bit, from per-word
// prefix counts. Cells are processed in runs of SF_CPT consecutive cells per
// thread; a cell's first triangle index comes from per-block prefix counts.
#include "vdm_internal.hpp"

namespace vdm {
namespace {

// ------------------------------------------------------------------ case table
// The 12 cube edges in ascending order of their global edge id: by axis, then by
// the lower corner (di, dj, dk) in row-major order.
struct CubeEdge {
  int d[3];
  int a;
};
constexpr CubeEdge kEdge[12] = {{{0, 0, 0}, 0}, {{0, 0, 1}, 0}, {{0, 1, 0}, 0}, {{0, 1, 1}, 0},
                                {{0, 0, 0}, 1}, {{0, 0, 1}, 1}, {{1, 0, 0}, 1}, {{1, 0, 1}, 1},
                                {{0, 0, 0}, 2}, {{0, 1, 0}, 2}, {{1, 0, 0}, 2}, {{1, 1, 0}, 2}};

struct McCase {
  unsigned char ntri;
  unsigned char e[5][3];  // per triangle vertex: axis << 3 | di << 2 | dj << 1 | dk of its cube edge
};
struct McTable {
  McCase c[256];
};

// corner (di, dj, dk) <-> case bit 4 di + 2 dj + dk
constexpr bool corner_in(int cs, int di, int dj, int dk) { return (cs >> (4 * di + 2 * dj + dk)) & 1; }
constexpr bool edge_touches(const CubeEdge& e, const int (&c)[3]) {
  for (int f = 0; f < 3; ++f)
    if (f != e.a && e.d[f] != c[f]) return false;
  return true;  // c is the lower or the upper end point
}
constexpr bool edge_crosses(int cs, const CubeEdge& e) {
  int u[3] = {e.d[0], e.d[1], e.d[2]};
  u[e.a] = 1;
  return corner_in(cs, e.d[0], e.d[1], e.d[2]) != corner_in(cs, u[0], u[1], u[2]);
}
constexpr bool share_face(const CubeEdge& x, const CubeEdge& y) {
  for (int f = 0; f < 3; ++f)
    if (f != x.a && f != y.a && x.d[f] == y.d[f]) return true;
  return false;
}

struct Vec3 {
  int v[3];
};
constexpr int dot3(const Vec3& x, const Vec3& y) { return x.v[0] * y.v[0] + x.v[1] * y.v[1] + x.v[2] * y.v[2]; }
constexpr Vec3 cross3(const Vec3& x, const Vec3& y) {
  return Vec3{{x.v[1] * y.v[2] - x.v[2] * y.v[1], x.v[2] * y.v[0] - x.v[0] * y.v[2], x.v[0] * y.v[1] - x.v[1] * y.v[0]}};
}
// twice the midpoint of a cube edge
constexpr Vec3 mid2(const CubeEdge& e) {
  Vec3 m{{2 * e.d[0], 2 * e.d[1], 2 * e.d[2]}};
  m.v[e.a] += 1;
  return m;
}

// Not constexpr: reaching it stops the compile-time evaluation of the table.
inline void table_error() {}

// Directs the segment between local edges ea and eb on the face with outward
// normal n so that (seen from outside the cube) the surface normal points along
// g, the in-face direction from the inside corners to the outside ones.
constexpr void put_segment(int (&nxt)[12], int ea, int eb, const Vec3& g, const Vec3& n) {
  const Vec3 t = cross3(g, n);
  const Vec3 ma = mid2(kEdge[ea]), mb = mid2(kEdge[eb]);
  const Vec3 d{{mb.v[0] - ma.v[0], mb.v[1] - ma.v[1], mb.v[2] - ma.v[2]}};
  const int dt = dot3(d, t);
  const int from = dt > 0 ? ea : eb, to = dt > 0 ? eb : ea;
  if (dt == 0 || nxt[from] >= 0) table_error();  // (cannot happen)
  nxt[from] = to;
}

constexpr McCase build_case(int cs) {
  int nxt[12] = {-1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1};
  for (int f = 0; f < 3; ++f)
    for (int s = 0; s < 2; ++s) {
      Vec3 n{{0, 0, 0}};
      n.v[f] = 2 * s - 1;
      int corners[4][3] = {};
      int nc = 0;
      for (int di = 0; di < 2; ++di)
        for (int dj = 0; dj < 2; ++dj)
          for (int dk = 0; dk < 2; ++dk) {
            const int c[3] = {di, dj, dk};
            if (c[f] != s) continue;
            corners[nc][0] = di, corners[nc][1] = dj, corners[nc][2] = dk;
            ++nc;
          }
      int fe[4] = {}, nfe = 0, ce[4] = {}, ncross = 0;
      for (int e = 0; e < 12; ++e)
        if (kEdge[e].a != f && kEdge[e].d[f] == s) {
          fe[nfe++] = e;
          if (edge_crosses(cs, kEdge[e])) ce[ncross++] = e;
        }
      Vec3 sum_in{{0, 0, 0}}, sum_out{{0, 0, 0}}, sum_all{{0, 0, 0}};
      int n_in = 0, n_out = 0;
      for (int q = 0; q < 4; ++q) {
        const bool in = corner_in(cs, corners[q][0], corners[q][1], corners[q][2]);
        for (int x = 0; x < 3; ++x) {
          (in ? sum_in : sum_out).v[x] += corners[q][x];
          sum_all.v[x] += corners[q][x];
        }
        (in ? n_in : n_out) += 1;
      }
      if (ncross == 2) {
        // g ~ centroid(outside corners) - centroid(inside corners)
        const Vec3 g{{sum_out.v[0] * n_in - sum_in.v[0] * n_out, sum_out.v[1] * n_in - sum_in.v[1] * n_out,
                      sum_out.v[2] * n_in - sum_in.v[2] * n_out}};
        put_segment(nxt, ce[0], ce[1], g, n);
      } else if (ncross == 4) {
        // each inside corner cut off by the segment between its two face edges;
        // g ~ face centre - corner
        for (int q = 0; q < 4; ++q) {
          if (!corner_in(cs, corners[q][0], corners[q][1], corners[q][2])) continue;
          int two[2] = {}, m = 0;
          for (int e = 0; e < 4; ++e)
            if (edge_touches(kEdge[fe[e]], corners[q])) two[m++] = fe[e];
          const Vec3 g{{sum_all.v[0] - 4 * corners[q][0], sum_all.v[1] - 4 * corners[q][1],
                        sum_all.v[2] - 4 * corners[q][2]}};
          put_segment(nxt, two[0], two[1], g, n);
        }
      }
    }
  McCase out{};
  bool seen[12] = {};
  for (int e0 = 0; e0 < 12; ++e0) {  // loops in order of their smallest edge
    if (nxt[e0] < 0 || seen[e0]) continue;
    int loop[12] = {}, len = 0;
    for (int e = e0; !seen[e]; e = nxt[e]) {
      seen[e] = true;
      loop[len++] = e;
    }
    int apex = -1;
    for (int p = 0; p < len; ++p) {
      bool ok = true;
      for (int m = 2; m + 1 < len; ++m)
        if (share_face(kEdge[loop[p]], kEdge[loop[(p + m) % len]])) ok = false;
      if (ok && (apex < 0 || loop[p] < loop[apex])) apex = p;
    }
    if (apex < 0 || out.ntri + len - 2 > 5) table_error();  // (cannot happen)
    for (int m = 1; m + 1 < len; ++m) {
      const int le[3] = {loop[apex], loop[(apex + m) % len], loop[(apex + m + 1) % len]};
      for (int x = 0; x < 3; ++x) {
        const CubeEdge& e = kEdge[le[x]];
        out.e[out.ntri][x] = (unsigned char)(e.a << 3 | e.d[0] << 2 | e.d[1] << 1 | e.d[2]);
      }
      ++out.ntri;
    }
  }
  return out;
}

constexpr McTable build_table() {
  McTable t{};
  for (int cs = 0; cs < 256; ++cs) t.c[cs] = build_case(cs);
  return t;
}

__constant__ McTable kTable = build_table();

// ------------------------------------------------------------------ kernels
constexpr int SF_NT = 256;         // threads per block
constexpr int SF_CPT = 8;          // consecutive cells per thread
constexpr int SF_CPB = SF_NT * SF_CPT;
constexpr int SF_WPT = 8;          // edge words per thread in the word scan
constexpr int SF_WPB = SF_NT * SF_WPT;

__device__ __forceinline__ bool inside(float v) { return v < 0.f; }

__device__ __forceinline__ bool cell_listed(const uint8_t* mask, int R, int i, int j, int k) {
  return i >= 0 && j >= 0 && k >= 0 && i < R && j < R && k < R && mask[((int64_t)i * R + j) * R + k] != 0;
}

// Crossing-edge bits: wave m covers points 64 m .. 64 m + 63; lane 0..2 writes the
// wave's word of axis a at words[a * nwa + m]. With a cell mask, an edge counts
// only when one of the (up to 4) cells around it is listed.
__global__ __launch_bounds__(SF_NT) void sf_edges_kernel(const float* __restrict__ vol, int R,
                                                         const uint8_t* __restrict__ mask,
                                                         uint64_t* __restrict__ words, int64_t nwa) {
  const int P = R + 1;
  const int64_t NP = (int64_t)P * P * P;
  const int lane = threadIdx.x & 63;
  const int64_t waves = (int64_t)gridDim.x * (SF_NT / 64);
  for (int64_t m = ((int64_t)blockIdx.x * SF_NT + threadIdx.x) / 64; m < nwa; m += waves) {
    const int64_t p = 64 * m + lane;
    bool f0 = false, f1 = false, f2 = false;
    if (p < NP) {
      const int i = (int)(p / ((int64_t)P * P));
      const int r = (int)(p - (int64_t)i * P * P);
      const int j = r / P, k = r - j * P;
      const bool in = inside(vol[p]);
      if (i < R) f0 = in != inside(vol[p + (int64_t)P * P]);
      if (j < R) f1 = in != inside(vol[p + P]);
      if (k < R) f2 = in != inside(vol[p + 1]);
      if (mask) {
        // cells holding edge (p, a): lower corner p minus 0/1 along the other two axes
        if (f0) f0 = cell_listed(mask, R, i, j, k) || cell_listed(mask, R, i, j - 1, k) ||
                     cell_listed(mask, R, i, j, k - 1) || cell_listed(mask, R, i, j - 1, k - 1);
        if (f1) f1 = cell_listed(mask, R, i, j, k) || cell_listed(mask, R, i - 1, j, k) ||
                     cell_listed(mask, R, i, j, k - 1) || cell_listed(mask, R, i - 1, j, k - 1);
        if (f2) f2 = cell_listed(mask, R, i, j, k) || cell_listed(mask, R, i - 1, j, k) ||
                     cell_listed(mask, R, i, j - 1, k) || cell_listed(mask, R, i - 1, j - 1, k);
      }
    }
    const uint64_t b0 = __ballot(f0), b1 = __ballot(f1), b2 = __ballot(f2);
    if (lane < 3) words[lane * nwa + m] = lane == 0 ? b0 : (lane == 1 ? b1 : b2);
  }
}

// Exclusive prefix of v over the block's threads (thread order), plus the total.
__device__ __forceinline__ int64_t block_exclusive(int64_t v, int64_t* red, int64_t& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int64_t x = v;  // inclusive scan within the wave
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) red[w] = x;
  __syncthreads();
  int64_t before = 0;
  total = 0;
#pragma unroll
  for (int q = 0; q < SF_NT / 64; ++q) {
    if (q < w) before += red[q];
    total += red[q];
  }
  return before + x - v;
}

__global__ __launch_bounds__(SF_NT) void sf_word_sums_kernel(const uint64_t* __restrict__ words, int64_t n,
                                                             int64_t* __restrict__ part) {
  __shared__ int64_t red[SF_NT / 64];
  const int64_t base = (int64_t)blockIdx.x * SF_WPB + (int64_t)threadIdx.x * SF_WPT;
  int64_t c = 0;
#pragma unroll
  for (int q = 0; q < SF_WPT; ++q)
    if (base + q < n) c += __popcll(words[base + q]);
  int64_t total;
  block_exclusive(c, red, total);
  if (threadIdx.x == 0) part[blockIdx.x] = total;
}

// In-place exclusive scan of part[0 .. nb) by one block; the total goes to *total.
__global__ __launch_bounds__(SF_NT) void sf_scan_parts_kernel(int64_t* __restrict__ part, int64_t nb,
                                                              int64_t* __restrict__ total) {
  __shared__ int64_t red[SF_NT / 64];
  int64_t carry = 0;
  for (int64_t b0 = 0; b0 < nb; b0 += SF_NT) {
    const int64_t b = b0 + threadIdx.x;
    const int64_t v = b < nb ? part[b] : 0;
    int64_t t;
    const int64_t ex = block_exclusive(v, red, t);
    if (b < nb) part[b] = carry + ex;
    carry += t;
    __syncthreads();
  }
  if (threadIdx.x == 0) *total = carry;
}

// Per-word prefix (vertex id of the word's first set bit).
__global__ __launch_bounds__(SF_NT) void sf_word_prefix_kernel(const uint64_t* __restrict__ words, int64_t n,
                                                               const int64_t* __restrict__ part,
                                                               int32_t* __restrict__ prefix) {
  __shared__ int64_t red[SF_NT / 64];
  const int64_t base = (int64_t)blockIdx.x * SF_WPB + (int64_t)threadIdx.x * SF_WPT;
  int c[SF_WPT];
  int64_t s = 0;
#pragma unroll
  for (int q = 0; q < SF_WPT; ++q) {
    c[q] = base + q < n ? __popcll(words[base + q]) : 0;
    s += c[q];
  }
  int64_t total;
  int64_t off = part[blockIdx.x] + block_exclusive(s, red, total);
#pragma unroll
  for (int q = 0; q < SF_WPT; ++q)
    if (base + q < n) {
      prefix[base + q] = (int32_t)off;
      off += c[q];
    }
}

__device__ __forceinline__ int cell_case(const float* __restrict__ vol, int P, int64_t p0) {
  const int64_t PP = (int64_t)P * P;
  int cs = 0;
#pragma unroll
  for (int di = 0; di < 2; ++di)
#pragma unroll
    for (int dj = 0; dj < 2; ++dj)
#pragma unroll
      for (int dk = 0; dk < 2; ++dk)
        cs |= (int)inside(vol[p0 + di * PP + dj * P + dk]) << (4 * di + 2 * dj + dk);
  return cs;
}

// Triangle counts of cells c0 .. c0 + SF_CPT - 1 (0 outside the grid or the mask).
__device__ __forceinline__ void run_counts(const float* __restrict__ vol, int R, const uint8_t* __restrict__ mask,
                                           int64_t c0, int (&cs)[SF_CPT], int (&nt)[SF_CPT]) {
  const int P = R + 1;
  const int64_t NC = (int64_t)R * R * R;
#pragma unroll
  for (int q = 0; q < SF_CPT; ++q) {
    const int64_t c = c0 + q;
    cs[q] = 0;
    nt[q] = 0;
    if (c >= NC || (mask && !mask[c])) continue;
    const int i = (int)(c / ((int64_t)R * R));
    const int r = (int)(c - (int64_t)i * R * R);
    const int j = r / R, k = r - j * R;
    cs[q] = cell_case(vol, P, ((int64_t)i * P + j) * P + k);
    nt[q] = kTable.c[cs[q]].ntri;
  }
}

__global__ __launch_bounds__(SF_NT) void sf_cell_sums_kernel(const float* __restrict__ vol, int R,
                                                             const uint8_t* __restrict__ mask,
                                                             int64_t* __restrict__ part) {
  __shared__ int64_t red[SF_NT / 64];
  int cs[SF_CPT], nt[SF_CPT];
  run_counts(vol, R, mask, (int64_t)blockIdx.x * SF_CPB + (int64_t)threadIdx.x * SF_CPT, cs, nt);
  int64_t s = 0;
#pragma unroll
  for (int q = 0; q < SF_CPT; ++q) s += nt[q];
  int64_t total;
  block_exclusive(s, red, total);
  if (threadIdx.x == 0) part[blockIdx.x] = total;
}

// Vertex id of global edge (axis a, point p): rank of its bit.
__device__ __forceinline__ int32_t vertex_of(const uint64_t* __restrict__ words, const int32_t* __restrict__ prefix,
                                            int64_t nwa, int a, int64_t p) {
  const int64_t w = a * nwa + (p >> 6);
  const uint64_t below = words[w] & ((1ull << (p & 63)) - 1ull);
  return prefix[w] + __popcll(below);
}

__global__ __launch_bounds__(SF_NT) void sf_triangles_kernel(const float* __restrict__ vol, int R,
                                                             const uint8_t* __restrict__ mask,
                                                             const uint64_t* __restrict__ words,
                                                             const int32_t* __restrict__ prefix, int64_t nwa,
                                                             const int64_t* __restrict__ part,
                                                             int32_t* __restrict__ tris, int64_t max_tris) {
  __shared__ int64_t red[SF_NT / 64];
  const int P = R + 1;
  const int64_t PP = (int64_t)P * P;
  const int64_t c0 = (int64_t)blockIdx.x * SF_CPB + (int64_t)threadIdx.x * SF_CPT;
  int cs[SF_CPT], nt[SF_CPT];
  run_counts(vol, R, mask, c0, cs, nt);
  int64_t s = 0;
#pragma unroll
  for (int q = 0; q < SF_CPT; ++q) s += nt[q];
  int64_t total;
  int64_t t = part[blockIdx.x] + block_exclusive(s, red, total);
  for (int q = 0; q < SF_CPT; ++q) {
    if (nt[q] == 0) continue;
    const int64_t c = c0 + q;
    const int i = (int)(c / ((int64_t)R * R));
    const int r = (int)(c - (int64_t)i * R * R);
    const int j = r / R, k = r - j * R;
    const int64_t p0 = ((int64_t)i * P + j) * P + k;
    const McCase& mc = kTable.c[cs[q]];
    for (int m = 0; m < mc.ntri; ++m, ++t) {
      if (t >= max_tris) continue;
      int32_t v[3];
#pragma unroll
      for (int x = 0; x < 3; ++x) {
        const int code = mc.e[m][x];
        v[x] = vertex_of(words, prefix, nwa, code >> 3, p0 + ((code >> 2) & 1) * PP + ((code >> 1) & 1) * P + (code & 1));
      }
      tris[3 * t + 0] = v[0];
      tris[3 * t + 1] = v[1];
      tris[3 * t + 2] = v[2];
    }
  }
}

// Vertex positions (and optionally edge ids), one thread per point.
__global__ __launch_bounds__(SF_NT) void sf_vertices_kernel(const float* __restrict__ vol, int R,
                                                            const uint64_t* __restrict__ words,
                                                            const int32_t* __restrict__ prefix, int64_t nwa,
                                                            float* __restrict__ verts, int64_t max_verts,
                                                            int64_t* __restrict__ vert_edges) {
  const int P = R + 1;
  const int64_t PP = (int64_t)P * P, NP = PP * P;
  const float h = 2.0f / (float)R;
  const int64_t stride = (int64_t)gridDim.x * SF_NT;
  for (int64_t p = (int64_t)blockIdx.x * SF_NT + threadIdx.x; p < 64 * nwa; p += stride) {
    if (p >= NP) continue;
    const int64_t m = p >> 6;
    const uint64_t low = (1ull << (p & 63)) - 1ull;
#pragma unroll
    for (int a = 0; a < 3; ++a) {
      const uint64_t w = words[a * nwa + m];
      if (!((w >> (p & 63)) & 1ull)) continue;
      const int64_t vid = prefix[a * nwa + m] + __popcll(w & low);
      if (vid >= max_verts) continue;
      const int i = (int)(p / PP);
      const int r = (int)(p - (int64_t)i * PP);
      const int j = r / P, k = r - j * P;
      const int64_t step = a == 0 ? PP : (a == 1 ? (int64_t)P : 1);
      const float v0 = vol[p], v1 = vol[p + step];
      const float t = v0 / (v0 - v1);
      float x = fmaf((float)i, h, -1.f), y = fmaf((float)j, h, -1.f), z = fmaf((float)k, h, -1.f);
      if (a == 0) x = fmaf(t, h, x);
      if (a == 1) y = fmaf(t, h, y);
      if (a == 2) z = fmaf(t, h, z);
      verts[3 * vid + 0] = x;
      verts[3 * vid + 1] = y;
      verts[3 * vid + 2] = z;
      if (vert_edges) vert_edges[vid] = a * NP + p;
    }
  }
}

int64_t grid_blocks(int64_t work, int64_t per_block, int64_t cap) {
  int64_t g = (work + per_block - 1) / per_block;
  if (g > cap) g = cap;
  return g < 1 ? 1 : g;
}

}  // namespace

SurfaceWs surface_ws_layout(int R) {
  const int64_t P = R + 1, NP = P * P * P, NC = (int64_t)R * R * R;
  SurfaceWs w{};
  w.nwa = (NP + 63) / 64;
  w.nwords = 3 * w.nwa;
  w.nwb = (w.nwords + SF_WPB - 1) / SF_WPB;
  w.ncb = (NC + SF_CPB - 1) / SF_CPB;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) / 256 * 256;
    return o;
  };
  w.off_words = take(8 * w.nwords);
  w.off_prefix = take(4 * w.nwords);
  w.off_wpart = take(8 * w.nwb);
  w.off_cpart = take(8 * w.ncb);
  w.bytes = off;
  return w;
}

hipError_t launch_surface(const float* vol, int R, const uint8_t* mask, float* verts, int64_t max_verts,
                          int32_t* tris, int64_t max_tris, int64_t* vert_edges, int64_t* counts, char* ws,
                          hipStream_t s) {
  const SurfaceWs w = surface_ws_layout(R);
  uint64_t* words = reinterpret_cast<uint64_t*>(ws + w.off_words);
  int32_t* prefix = reinterpret_cast<int32_t*>(ws + w.off_prefix);
  int64_t* wpart = reinterpret_cast<int64_t*>(ws + w.off_wpart);
  int64_t* cpart = reinterpret_cast<int64_t*>(ws + w.off_cpart);
  const int64_t cus = dev_info().cus;
  hipLaunchKernelGGL(sf_edges_kernel, dim3((unsigned)grid_blocks(w.nwa, SF_NT / 64, 64 * cus)), dim3(SF_NT), 0, s,
                     vol, R, mask, words, w.nwa);
  hipLaunchKernelGGL(sf_word_sums_kernel, dim3((unsigned)w.nwb), dim3(SF_NT), 0, s, words, w.nwords, wpart);
  hipLaunchKernelGGL(sf_scan_parts_kernel, dim3(1), dim3(SF_NT), 0, s, wpart, w.nwb, counts);
  hipLaunchKernelGGL(sf_word_prefix_kernel, dim3((unsigned)w.nwb), dim3(SF_NT), 0, s, words, w.nwords, wpart, prefix);
  hipLaunchKernelGGL(sf_cell_sums_kernel, dim3((unsigned)w.ncb), dim3(SF_NT), 0, s, vol, R, mask, cpart);
  hipLaunchKernelGGL(sf_scan_parts_kernel, dim3(1), dim3(SF_NT), 0, s, cpart, w.ncb, counts + 1);
  hipLaunchKernelGGL(sf_triangles_kernel, dim3((unsigned)w.ncb), dim3(SF_NT), 0, s, vol, R, mask, words, prefix,
                     w.nwa, cpart, tris, max_tris);
  hipLaunchKernelGGL(sf_vertices_kernel, dim3((unsigned)grid_blocks(64 * w.nwa, SF_NT, 64 * cus)), dim3(SF_NT), 0, s,
                     vol, R, words, prefix, w.nwa, verts, max_verts, vert_edges);
  return hipGetLastError();
}

}  // namespace vdm
