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
// GPU layout: a point row (i, j) is cut into pieces of 63 points, k = 63 kc + l,
// l < 63; one 64-bit word per piece holds one bit per point (bit 63 unused), so a
// wave of 64 lanes reads a piece plus the next point and writes whole words.
// Per axis a plane of such words marks the crossing edges (bit = lower end
// point); a vertex id is the rank of its bit over the planes in order, from
// per-word prefix counts. A fourth plane holds the inside bits (bit 63 = the
// next piece's first point). One pass over the volume (each wave walks a column
// of pieces along i, so every value is loaded about twice) writes the planes and
// the triangle count of every piece; a cell's first triangle index comes from
// the prefix of those counts.
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
// Point and vertex indices fit 32 bits: R <= 893 keeps 3 (R+1)^3 below 2^31.
constexpr int SF_NT = 256;   // threads per block (4 waves)
constexpr int SF_PW = 63;    // points per piece
constexpr int SF_IC = 16;    // pieces along i per wave in the volume pass
constexpr int SF_TPW = 16;   // pieces per wave in the triangle and vertex passes
constexpr int SF_WPT = 8;    // values per thread in the block sums / prefixes
constexpr int SF_WPB = SF_NT * SF_WPT;
constexpr int SF_PPT = 16;   // partial sums per thread in the one-block scan

__device__ __forceinline__ bool inside(float v) { return v < 0.f; }

__device__ __forceinline__ bool cell_listed(const uint8_t* mask, int R, int i, int j, int k) {
  return i >= 0 && j >= 0 && k >= 0 && i < R && j < R && k < R && mask[(i * R + j) * R + k] != 0;
}

// (the readlane builtin moves 32 bits)
__device__ __forceinline__ uint64_t readlane64(uint64_t x, int lane) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, lane);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), lane);
  return (uint64_t)hi << 32 | lo;
}

__device__ __forceinline__ int pieces_per_row(int P) { return (P + SF_PW - 1) / SF_PW; }

__device__ __forceinline__ void load_ntri(unsigned char* ntri) {
  for (int c = threadIdx.x; c < 256; c += SF_NT) ntri[c] = kTable.c[c].ntri;
  __syncthreads();
}

// Case of cell (i, j, k) of lane l < 63 from the inside words of its four corner
// rows (bits l and l + 1).
__device__ __forceinline__ int cell_case(uint64_t b00, uint64_t b01, uint64_t b10, uint64_t b11, int l) {
  return (int)((b00 >> l) & 3ull) | (int)((b01 >> l) & 3ull) << 2 | (int)((b10 >> l) & 3ull) << 4 |
         (int)((b11 >> l) & 3ull) << 6;
}

// The volume pass. Block b covers rows j = 4 jg + wave, piece column kc, and
// pieces i = SF_IC ic .. SF_IC ic + SF_IC - 1 (b = (jg * KC + kc) * NIC + ic). Per
// piece (i, j, kc): the crossing-edge words of the three axes (planes[a * nwp +
// piece]), the inside word (ins[piece]) and the triangle count of its cells
// (tcnt[piece]). With a cell mask an edge counts only when one of the (up to 4)
// cells around it is listed, and only listed cells have triangles.
template <bool MASKED>
__global__ __launch_bounds__(SF_NT) void sf_points_kernel(const float* __restrict__ vol, int R,
                                                          const uint8_t* __restrict__ mask,
                                                          uint64_t* __restrict__ planes, uint64_t* __restrict__ ins,
                                                          int32_t* __restrict__ tcnt) {
  __shared__ unsigned char ntri[256];
  load_ntri(ntri);
  const int P = R + 1, KC = pieces_per_row(P), nwp = P * P * KC, NIC = (P + SF_IC - 1) / SF_IC;
  const int l = threadIdx.x & 63;
  const int ic = blockIdx.x % NIC, rest = blockIdx.x / NIC;
  const int kc = rest % KC, jg = rest / KC;
  const int j = __builtin_amdgcn_readfirstlane(4 * jg + (threadIdx.x >> 6));
  if (j >= P) return;  // (no barrier follows)
  const int i0 = ic * SF_IC;
  const int k = SF_PW * kc + l;
  const bool ok = k < P;
  const int kk = min(k, R), j1 = min(j + 1, R);
  // rows (i, j) and (i, j+1) for i = i0 .. i0 + SF_IC (clamped to the grid), all loads first
  float a[SF_IC + 1], b[SF_IC + 1];
#pragma unroll
  for (int t = 0; t <= SF_IC; ++t) {
    const int i = min(i0 + t, R);
    a[t] = vol[(i * P + j) * P + kk];
    b[t] = vol[(i * P + j1) * P + kk];
  }
  // lane t keeps the words of piece i0 + t and stores them after the walk (one
  // store instruction per output instead of one per piece)
  uint64_t ox = 0, oy = 0, oz = 0, oi = 0;
  int ocnt = 0;
#pragma unroll
  for (int t = 0; t < SF_IC; ++t) {
    const int i = i0 + t;  // (rows past R: clamped loads, nothing stored)
    const bool in00 = ok && inside(a[t]), in01 = ok && inside(b[t]), in10 = ok && inside(a[t + 1]),
               in11 = ok && inside(b[t + 1]);
    const uint64_t b00 = __ballot(in00), b01 = __ballot(in01), b10 = __ballot(in10), b11 = __ballot(in11);
    const bool own = ok && l < SF_PW;
    bool fx = own && i < R && in00 != in10;
    bool fy = own && j < R && in00 != in01;
    bool fz = own && k < R && in00 != (bool)((b00 >> (l + 1)) & 1ull);
    if constexpr (MASKED) {
      // cells holding the edge: lower corner (i, j, k) minus 0/1 along the other two axes
      if (fx) fx = cell_listed(mask, R, i, j, k) || cell_listed(mask, R, i, j - 1, k) ||
                   cell_listed(mask, R, i, j, k - 1) || cell_listed(mask, R, i, j - 1, k - 1);
      if (fy) fy = cell_listed(mask, R, i, j, k) || cell_listed(mask, R, i - 1, j, k) ||
                   cell_listed(mask, R, i, j, k - 1) || cell_listed(mask, R, i - 1, j, k - 1);
      if (fz) fz = cell_listed(mask, R, i, j, k) || cell_listed(mask, R, i - 1, j, k) ||
                   cell_listed(mask, R, i, j - 1, k) || cell_listed(mask, R, i - 1, j - 1, k);
    }
    const uint64_t bx = __ballot(fx), by = __ballot(fy), bz = __ballot(fz);
    // cell (i, j, k): corners in rows (i|i+1, j|j+1), points k, k+1; at most 5
    // triangles, so the piece's sum comes from three ballots of the count's bits
    int nt = 0;
    if (own && i < R && j < R && k < R && (!MASKED || mask[(i * R + j) * R + k] != 0))
      nt = ntri[cell_case(b00, b01, b10, b11, l)];
    const int sum = __popcll(__ballot(nt & 1)) + 2 * __popcll(__ballot(nt & 2)) + 4 * __popcll(__ballot(nt & 4));
    if (l == t) {
      ox = bx;
      oy = by;
      oz = bz;
      oi = b00;
      ocnt = sum;
    }
  }
  if (l < SF_IC && i0 + l <= R) {
    const int piece = ((i0 + l) * P + j) * KC + kc;
    planes[piece] = ox;
    planes[nwp + piece] = oy;
    planes[2 * nwp + piece] = oz;
    ins[piece] = oi;
    tcnt[piece] = ocnt;
  }
}

__device__ __forceinline__ int64_t count_of(const uint64_t* x, int i) { return __popcll(x[i]); }
__device__ __forceinline__ int64_t count_of(const int32_t* x, int i) { return x[i]; }

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

// Per-block sums of count_of(x, i), i < n (blocks of SF_WPB entries).
template <typename X>
__global__ __launch_bounds__(SF_NT) void sf_block_sums_kernel(const X* __restrict__ x, int n,
                                                              int64_t* __restrict__ part) {
  __shared__ int64_t red[SF_NT / 64];
  const int base = blockIdx.x * SF_WPB + threadIdx.x * SF_WPT;
  int64_t c = 0;
#pragma unroll
  for (int q = 0; q < SF_WPT; ++q)
    if (base + q < n) c += count_of(x, base + q);
  int64_t total;
  block_exclusive(c, red, total);
  if (threadIdx.x == 0) part[blockIdx.x] = total;
}

// In-place exclusive scan of part[0 .. nb) by one block; the total goes to *total.
__global__ __launch_bounds__(SF_NT) void sf_scan_parts_kernel(int64_t* __restrict__ part, int nb,
                                                              int64_t* __restrict__ total) {
  __shared__ int64_t red[SF_NT / 64];
  int64_t carry = 0;
  for (int b0 = 0; b0 < nb; b0 += SF_NT * SF_PPT) {
    const int base = b0 + threadIdx.x * SF_PPT;
    int64_t v[SF_PPT], s = 0;
#pragma unroll
    for (int q = 0; q < SF_PPT; ++q) {
      v[q] = base + q < nb ? part[base + q] : 0;
      s += v[q];
    }
    int64_t t;
    int64_t run = carry + block_exclusive(s, red, t);
#pragma unroll
    for (int q = 0; q < SF_PPT; ++q)
      if (base + q < nb) {
        part[base + q] = run;
        run += v[q];
      }
    carry += t;
    __syncthreads();
  }
  if (threadIdx.x == 0) *total = carry;
}

// Exclusive prefix of count_of(x, i) (part: the scanned block sums).
template <typename X, typename Y>
__global__ __launch_bounds__(SF_NT) void sf_prefix_kernel(const X* __restrict__ x, int n,
                                                          const int64_t* __restrict__ part, Y* __restrict__ prefix) {
  __shared__ int64_t red[SF_NT / 64];
  const int base = blockIdx.x * SF_WPB + threadIdx.x * SF_WPT;
  int64_t c[SF_WPT];
  int64_t s = 0;
#pragma unroll
  for (int q = 0; q < SF_WPT; ++q) {
    c[q] = base + q < n ? count_of(x, base + q) : 0;
    s += c[q];
  }
  int64_t total;
  int64_t off = part[blockIdx.x] + block_exclusive(s, red, total);
#pragma unroll
  for (int q = 0; q < SF_WPT; ++q)
    if (base + q < n) {
      prefix[base + q] = (Y)off;
      off += c[q];
    }
}

// Vertex id of the edge along axis a from point (row, k): rank of its bit.
__device__ __forceinline__ int32_t vertex_of(const uint64_t* __restrict__ planes, const int32_t* __restrict__ vpre,
                                            int nwp, int KC, int a, int row, int k) {
  const int kc = k / SF_PW, l = k - kc * SF_PW;
  const int w = a * nwp + row * KC + kc;
  return vpre[w] + __popcll(planes[w] & ((1ull << l) - 1ull));
}

// Triangles: a wave per SF_TPW pieces, skipping those without triangles. A lane
// with triangles fetches the vertex ids of all 12 edges of its cell (independent
// loads, in flight together), keeps them in LDS and writes its triangles from the
// case table.
template <bool MASKED>
__global__ __launch_bounds__(SF_NT) void sf_triangles_kernel(int R, const uint8_t* __restrict__ mask,
                                                             const uint64_t* __restrict__ planes,
                                                             const uint64_t* __restrict__ ins,
                                                             const int32_t* __restrict__ vpre,
                                                             const int32_t* __restrict__ tcnt,
                                                             const int64_t* __restrict__ tpre,
                                                             int32_t* __restrict__ tris, int64_t max_tris) {
  __shared__ McCase tab[256];
  __shared__ int32_t vid_lds[12][SF_NT];
  for (int c = threadIdx.x; c < 256; c += SF_NT) tab[c] = kTable.c[c];
  __syncthreads();
  const int P = R + 1, KC = pieces_per_row(P), nwp = P * P * KC;
  const int l = threadIdx.x & 63;
  const int p0 = __builtin_amdgcn_readfirstlane((blockIdx.x * SF_NT + threadIdx.x) >> 6) * SF_TPW;
  // the triangle counts of the wave's pieces, one per lane, in one load
  const int cnt_l = l < SF_TPW && p0 + l < nwp ? tcnt[p0 + l] : 0;
  for (int q = 0; q < SF_TPW; ++q) {
    const int piece = p0 + q;
    if (__builtin_amdgcn_readlane(cnt_l, q) == 0) continue;  // (wave-uniform; 0 past the end)
    const int row = piece / KC, kc = piece - row * KC;
    const int i = row / P, j = row - i * P;
    const int k = SF_PW * kc + l;
    const uint64_t b00 = ins[piece], b01 = ins[piece + KC], b10 = ins[piece + P * KC], b11 = ins[piece + P * KC + KC];
    const int cs = cell_case(b00, b01, b10, b11, l);
    const int nt = l < SF_PW && k < R && (!MASKED || mask[(i * R + j) * R + k] != 0) ? tab[cs].ntri : 0;
    int x = nt;  // inclusive scan over the piece's cells (lane order = cell order)
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o);
      if (l >= o) x += y;
    }
    if (nt == 0) continue;
    int64_t u = tpre[piece] + x - nt;
    // vertex ids of the cell's 12 edges (edges that do not cross give unused values)
#pragma unroll
    for (int e = 0; e < 12; ++e) {
      // edge e: axis a = e / 4, offsets o1, o2 along the other two axes (in axis order)
      const int a = e >> 2, o1 = (e >> 1) & 1, o2 = e & 1;
      const int di = a == 0 ? 0 : o1, dj = a == 0 ? o1 : (a == 1 ? 0 : o2), dk = a == 2 ? 0 : o2;
      vid_lds[e][threadIdx.x] = vertex_of(planes, vpre, nwp, KC, a, row + di * P + dj, k + dk);
    }
    const McCase& mc = tab[cs];
    for (int m = 0; m < nt; ++m, ++u) {
      if (u >= max_tris) continue;
#pragma unroll
      for (int x3 = 0; x3 < 3; ++x3) {
        const int code = mc.e[m][x3];  // axis << 3 | di << 2 | dj << 1 | dk
        const int a = code >> 3;
        const int o1 = a == 0 ? (code >> 1) & 1 : (code >> 2) & 1;
        const int o2 = a == 2 ? (code >> 1) & 1 : code & 1;
        tris[3 * u + x3] = vid_lds[4 * a + 2 * o1 + o2][threadIdx.x];
      }
    }
  }
}

// Vertex positions (and optionally edge ids): a wave per SF_TPW pieces, all three axes.
__global__ __launch_bounds__(SF_NT) void sf_vertices_kernel(const float* __restrict__ vol, int R,
                                                            const uint64_t* __restrict__ planes,
                                                            const int32_t* __restrict__ vpre,
                                                            float* __restrict__ verts, int64_t max_verts,
                                                            int64_t* __restrict__ vert_edges) {
  const int P = R + 1, PP = P * P, NP = PP * P, KC = pieces_per_row(P), nwp = PP * KC;
  const float h = 2.0f / (float)R;
  const int l = threadIdx.x & 63;
  const int p0 = __builtin_amdgcn_readfirstlane((blockIdx.x * SF_NT + threadIdx.x) >> 6) * SF_TPW;
  // the three words of each of the wave's pieces, lane 3 u + a = axis a of piece p0 + u, in one load
  const int pl = p0 + l / 3;
  const uint64_t word_l = l < 3 * SF_TPW && pl < nwp ? planes[(l % 3) * nwp + pl] : 0ull;
  for (int u = 0; u < SF_TPW; ++u) {
    const int piece = p0 + u;
    const uint64_t w0 = readlane64(word_l, 3 * u), w1 = readlane64(word_l, 3 * u + 1),
                   w2 = readlane64(word_l, 3 * u + 2);  // wave-uniform (0 past the end)
    if ((w0 | w1 | w2) == 0) continue;
    if (!((w0 | w1 | w2) >> l & 1ull)) continue;
    const int row = piece / KC, kc = piece - row * KC;
    const int i = row / P, j = row - i * P;
    const int k = SF_PW * kc + l;
    const int p = row * P + k;
    const uint64_t low = (1ull << l) - 1ull;
    const float v0 = vol[p];
    const float bx = fmaf((float)i, h, -1.f), by = fmaf((float)j, h, -1.f), bz = fmaf((float)k, h, -1.f);
#pragma unroll
    for (int a = 0; a < 3; ++a) {
      const uint64_t w = a == 0 ? w0 : (a == 1 ? w1 : w2);
      if (!((w >> l) & 1ull)) continue;
      const int64_t vid = vpre[a * nwp + piece] + __popcll(w & low);
      if (vid >= max_verts) continue;
      const float v1 = vol[p + (a == 0 ? PP : (a == 1 ? P : 1))];
      const float t = v0 / (v0 - v1);
      verts[3 * vid + 0] = a == 0 ? fmaf(t, h, bx) : bx;
      verts[3 * vid + 1] = a == 1 ? fmaf(t, h, by) : by;
      verts[3 * vid + 2] = a == 2 ? fmaf(t, h, bz) : bz;
      if (vert_edges) vert_edges[vid] = (int64_t)a * NP + p;
    }
  }
}

int grid_blocks(int64_t work, int64_t per_block, int64_t cap) {
  int64_t g = (work + per_block - 1) / per_block;
  if (g > cap) g = cap;
  return g < 1 ? 1 : (int)g;
}

}  // namespace

SurfaceWs surface_ws_layout(int R) {
  const int64_t P = R + 1, KC = (P + SF_PW - 1) / SF_PW;
  SurfaceWs w{};
  w.nwa = P * P * KC;  // words per plane (one per piece)
  w.nwords = 3 * w.nwa;
  w.nwb = (w.nwords + SF_WPB - 1) / SF_WPB;
  w.ncb = (w.nwa + SF_WPB - 1) / SF_WPB;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) / 256 * 256;
    return o;
  };
  w.off_words = take(8 * w.nwords);
  w.off_ins = take(8 * w.nwa);
  w.off_prefix = take(4 * w.nwords);
  w.off_tcnt = take(4 * w.nwa);
  w.off_tpre = take(8 * w.nwa);
  w.off_wpart = take(8 * w.nwb);
  w.off_cpart = take(8 * w.ncb);
  w.bytes = off;
  return w;
}

hipError_t launch_surface(const float* vol, int R, const uint8_t* mask, float* verts, int64_t max_verts,
                          int32_t* tris, int64_t max_tris, int64_t* vert_edges, int64_t* counts, char* ws,
                          hipStream_t s) {
  const SurfaceWs w = surface_ws_layout(R);
  uint64_t* planes = reinterpret_cast<uint64_t*>(ws + w.off_words);
  uint64_t* ins = reinterpret_cast<uint64_t*>(ws + w.off_ins);
  int32_t* vpre = reinterpret_cast<int32_t*>(ws + w.off_prefix);
  int32_t* tcnt = reinterpret_cast<int32_t*>(ws + w.off_tcnt);
  int64_t* tpre = reinterpret_cast<int64_t*>(ws + w.off_tpre);
  int64_t* wpart = reinterpret_cast<int64_t*>(ws + w.off_wpart);
  int64_t* cpart = reinterpret_cast<int64_t*>(ws + w.off_cpart);
  const int P = R + 1, KC = (P + SF_PW - 1) / SF_PW, NIC = (P + SF_IC - 1) / SF_IC;
  const int nwp = (int)w.nwa, nwords = (int)w.nwords, nwb = (int)w.nwb, ncb = (int)w.ncb;
  const int gp = ((P + 3) / 4) * KC * NIC;
  if (mask)
    hipLaunchKernelGGL(sf_points_kernel<true>, dim3(gp), dim3(SF_NT), 0, s, vol, R, mask, planes, ins, tcnt);
  else
    hipLaunchKernelGGL(sf_points_kernel<false>, dim3(gp), dim3(SF_NT), 0, s, vol, R, mask, planes, ins, tcnt);
  hipLaunchKernelGGL(sf_block_sums_kernel<uint64_t>, dim3(nwb), dim3(SF_NT), 0, s, planes, nwords, wpart);
  hipLaunchKernelGGL(sf_scan_parts_kernel, dim3(1), dim3(SF_NT), 0, s, wpart, nwb, counts);
  hipLaunchKernelGGL((sf_prefix_kernel<uint64_t, int32_t>), dim3(nwb), dim3(SF_NT), 0, s, planes, nwords, wpart, vpre);
  hipLaunchKernelGGL(sf_block_sums_kernel<int32_t>, dim3(ncb), dim3(SF_NT), 0, s, tcnt, nwp, cpart);
  hipLaunchKernelGGL(sf_scan_parts_kernel, dim3(1), dim3(SF_NT), 0, s, cpart, ncb, counts + 1);
  hipLaunchKernelGGL((sf_prefix_kernel<int32_t, int64_t>), dim3(ncb), dim3(SF_NT), 0, s, tcnt, nwp, cpart, tpre);
  const int gt = grid_blocks(nwp, SF_TPW * (SF_NT / 64), INT32_MAX);
  if (mask)
    hipLaunchKernelGGL(sf_triangles_kernel<true>, dim3(gt), dim3(SF_NT), 0, s, R, mask, planes, ins, vpre, tcnt, tpre,
                       tris, max_tris);
  else
    hipLaunchKernelGGL(sf_triangles_kernel<false>, dim3(gt), dim3(SF_NT), 0, s, R, mask, planes, ins, vpre, tcnt, tpre,
                       tris, max_tris);
  hipLaunchKernelGGL(sf_vertices_kernel, dim3(grid_blocks(nwp, SF_TPW * (SF_NT / 64), INT32_MAX)), dim3(SF_NT), 0, s,
                     vol, R,
                     planes, vpre, verts, max_verts, vert_edges);
  return hipGetLastError();
}

VDM_DEBUG_READER(debug_take_surface)

}  // namespace vdm
