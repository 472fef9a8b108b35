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
// Every index fits 32 bits: R <= 893 keeps 3 (R+1)^3 below 2^31.
constexpr int SF_NT = 256;              // threads per block (4 waves)
// Cells go by row pieces: a piece is 64 consecutive cells (i, j, 64 kc .. 64 kc + 63)
// of one row, one per lane (the last piece of a row is ragged); a wave takes SF_IPW
// consecutive pieces, a block SF_PPB.
constexpr int SF_IPW = 8;
constexpr int SF_PPB = SF_IPW * (SF_NT / 64);
constexpr int SF_WPT = 8;               // edge words per thread in the word scan
constexpr int SF_WPB = SF_NT * SF_WPT;
constexpr int SF_PPT = 16;              // partial sums per thread in the one-block scan

__device__ __forceinline__ bool inside(float v) { return v < 0.f; }

__device__ __forceinline__ bool cell_listed(const uint8_t* mask, int R, int i, int j, int k) {
  return i >= 0 && j >= 0 && k >= 0 && i < R && j < R && k < R && mask[(i * R + j) * R + k] != 0;
}

// Crossing-edge bits and inside bits: wave m covers points 64 m .. 64 m + 63;
// lanes 0..2 write the wave's word of each axis plane (words[a * nwa + m]),
// lane 3 the inside bits (ins[m]). With a cell mask an edge counts only when one
// of the (up to 4) cells around it is listed.
__global__ __launch_bounds__(SF_NT) void sf_edges_kernel(const float* __restrict__ vol, int R,
                                                         const uint8_t* __restrict__ mask,
                                                         uint64_t* __restrict__ words, uint64_t* __restrict__ ins,
                                                         int nwa) {
  const int P = R + 1, PP = P * P, NP = PP * P;
  const int lane = threadIdx.x & 63;
  const int waves = gridDim.x * (SF_NT / 64);
  if (blockIdx.x == 0 && threadIdx.x == 0) ins[nwa] = 0;  // the spare word (read only for points past the grid)
  for (int m = __builtin_amdgcn_readfirstlane((blockIdx.x * SF_NT + threadIdx.x) >> 6); m < nwa; m += waves) {
    const int p = 64 * m + lane;
    // all four loads unconditional (clamped addresses), so they are in flight together
    const int pc = min(p, NP - 1);
    const float v = vol[pc], vi = vol[min(pc + PP, NP - 1)], vj = vol[min(pc + P, NP - 1)], vk = vol[pc + (pc + 1 < NP)];
    const int row = pc / P, k = pc - row * P;
    const int i = row / P, j = row - i * P;
    const bool ok = p < NP;
    const bool in = ok && inside(v);
    bool f0 = ok && i < R && inside(v) != inside(vi);
    bool f1 = ok && j < R && inside(v) != inside(vj);
    bool f2 = ok && k < R && inside(v) != inside(vk);
    {
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
    const uint64_t b0 = __ballot(f0), b1 = __ballot(f1), b2 = __ballot(f2), bi = __ballot(in);
    if (lane < 3) words[lane * nwa + m] = lane == 0 ? b0 : (lane == 1 ? b1 : b2);
    if (lane == 3) ins[m] = bi;
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

__global__ __launch_bounds__(SF_NT) void sf_word_sums_kernel(const uint64_t* __restrict__ words, int n,
                                                             int64_t* __restrict__ part) {
  __shared__ int64_t red[SF_NT / 64];
  const int base = blockIdx.x * SF_WPB + threadIdx.x * SF_WPT;
  int64_t c = 0;
#pragma unroll
  for (int q = 0; q < SF_WPT; ++q)
    if (base + q < n) c += __popcll(words[base + q]);
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

// Per-word prefix (vertex id of the word's first set bit).
__global__ __launch_bounds__(SF_NT) void sf_word_prefix_kernel(const uint64_t* __restrict__ words, int n,
                                                               const int64_t* __restrict__ part,
                                                               int32_t* __restrict__ prefix) {
  __shared__ int64_t red[SF_NT / 64];
  const int base = blockIdx.x * SF_WPB + threadIdx.x * SF_WPT;
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

// One row piece (see SF_IPW): its cells' cases, triangle counts and lower corners.
// The inside bits of the four corner rows come from two scalar word loads each
// (the piece's 65 points of a row span at most two words); ins has one spare
// word after the last one.
struct Piece {
  int cs, nt, p0;
};
__device__ __forceinline__ Piece piece_cell(const uint64_t* __restrict__ ins, int R, const uint8_t* __restrict__ mask,
                                            const unsigned char* ntri, int piece, int lane) {
  const int P = R + 1, KC = (R + 63) >> 6;
  Piece out{0, 0, 0};
  const int r = piece / KC, kc = piece - r * KC;  // wave-uniform
  if (r >= R * R) return out;
  const int i = r / R, j = r - i * R;
  const int k = 64 * kc + lane;
  int cs = 0;
#pragma unroll
  for (int di = 0; di < 2; ++di)
#pragma unroll
    for (int dj = 0; dj < 2; ++dj) {
      const int start = ((i + di) * P + (j + dj)) * P + 64 * kc;
      const int w = start >> 6, sh = start & 63;
      const uint64_t w0 = ins[w], w1 = ins[w + 1];
      const uint64_t lo = sh ? (w0 >> sh) | (w1 << (64 - sh)) : w0;
      const int b0 = (int)((lo >> lane) & 1ull);
      const int b1 = lane < 63 ? (int)((lo >> (lane + 1)) & 1ull) : (int)((w1 >> sh) & 1ull);
      cs |= b0 << (4 * di + 2 * dj) | b1 << (4 * di + 2 * dj + 1);
    }
  const int c = (i * R + j) * R + k;
  const bool ok = k < R && (!mask || mask[min(c, R * R * R - 1)] != 0);
  out.cs = cs;
  out.nt = ok ? ntri[cs] : 0;
  out.p0 = (i * P + j) * P + k;
  return out;
}

__device__ __forceinline__ void load_ntri(unsigned char* ntri) {
  for (int c = threadIdx.x; c < 256; c += SF_NT) ntri[c] = kTable.c[c].ntri;
  __syncthreads();
}

__device__ __forceinline__ int piece_of(int q) {
  return __builtin_amdgcn_readfirstlane(blockIdx.x * SF_PPB + (threadIdx.x >> 6) * SF_IPW + q);
}

__global__ __launch_bounds__(SF_NT) void sf_cell_sums_kernel(const uint64_t* __restrict__ ins, int R,
                                                             const uint8_t* __restrict__ mask,
                                                             int64_t* __restrict__ part) {
  __shared__ int64_t red[SF_NT / 64];
  __shared__ unsigned char ntri[256];
  load_ntri(ntri);
  const int lane = threadIdx.x & 63;
  int64_t s = 0;
#pragma unroll
  for (int q = 0; q < SF_IPW; ++q) s += piece_cell(ins, R, mask, ntri, piece_of(q), lane).nt;
  int64_t total;
  block_exclusive(s, red, total);
  if (threadIdx.x == 0) part[blockIdx.x] = total;
}

// Vertex id of global edge (axis a, point p): rank of its bit.
__device__ __forceinline__ int32_t vertex_of(const uint64_t* __restrict__ words, const int32_t* __restrict__ prefix,
                                            int nwa, int a, int p) {
  const int w = a * nwa + (p >> 6);
  const uint64_t below = words[w] & ((1ull << (p & 63)) - 1ull);
  return prefix[w] + __popcll(below);
}

__global__ __launch_bounds__(SF_NT) void sf_triangles_kernel(const uint64_t* __restrict__ ins, int R,
                                                             const uint8_t* __restrict__ mask,
                                                             const uint64_t* __restrict__ words,
                                                             const int32_t* __restrict__ prefix, int nwa,
                                                             const int64_t* __restrict__ part,
                                                             int32_t* __restrict__ tris, int64_t max_tris) {
  __shared__ int64_t red[SF_NT / 64];
  __shared__ unsigned char ntri[256];
  load_ntri(ntri);
  const int P = R + 1, PP = P * P;
  const int lane = threadIdx.x & 63;
  Piece pc[SF_IPW];
  int64_t s = 0;
#pragma unroll
  for (int q = 0; q < SF_IPW; ++q) {
    pc[q] = piece_cell(ins, R, mask, ntri, piece_of(q), lane);
    s += pc[q].nt;
  }
  // this wave's first triangle: block offset + the triangles of the waves before it
  int64_t total;
  const int64_t before = block_exclusive(s, red, total);
  int64_t t = part[blockIdx.x] + __shfl(before, 0);
#pragma unroll
  for (int q = 0; q < SF_IPW; ++q) {
    int x = pc[q].nt;  // inclusive scan over the piece's cells (lane order = cell order)
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    int64_t u = t + x - pc[q].nt;
    t += __shfl(x, 63);
    if (pc[q].nt == 0) continue;
    const McCase& mc = kTable.c[pc[q].cs];
    for (int m = 0; m < pc[q].nt; ++m, ++u) {
      if (u >= max_tris) continue;
      int32_t v[3];
#pragma unroll
      for (int x3 = 0; x3 < 3; ++x3) {
        const int code = mc.e[m][x3];
        v[x3] = vertex_of(words, prefix, nwa, code >> 3,
                          pc[q].p0 + ((code >> 2) & 1) * PP + ((code >> 1) & 1) * P + (code & 1));
      }
      tris[3 * u + 0] = v[0];
      tris[3 * u + 1] = v[1];
      tris[3 * u + 2] = v[2];
    }
  }
}

// Vertex positions (and optionally edge ids), one thread per point.
__global__ __launch_bounds__(SF_NT) void sf_vertices_kernel(const float* __restrict__ vol, int R,
                                                            const uint64_t* __restrict__ words,
                                                            const int32_t* __restrict__ prefix, int nwa,
                                                            float* __restrict__ verts, int64_t max_verts,
                                                            int64_t* __restrict__ vert_edges) {
  const int P = R + 1, PP = P * P, NP = PP * P;
  const float h = 2.0f / (float)R;
  const int lane = threadIdx.x & 63;
  const int waves = gridDim.x * (SF_NT / 64);
  for (int m = __builtin_amdgcn_readfirstlane((blockIdx.x * SF_NT + threadIdx.x) >> 6); m < nwa; m += waves) {
    const uint64_t w0 = words[m], w1 = words[nwa + m], w2 = words[2 * nwa + m];  // wave-uniform
    if ((w0 | w1 | w2) == 0) continue;
    const int p = 64 * m + lane;
    if (!((w0 | w1 | w2) >> lane & 1ull) || p >= NP) continue;
    const uint64_t low = (1ull << (p & 63)) - 1ull;
    const int row = p / P, k = p - row * P;
    const int i = row / P, j = row - i * P;
    const float v0 = vol[p];
    const float bx = fmaf((float)i, h, -1.f), by = fmaf((float)j, h, -1.f), bz = fmaf((float)k, h, -1.f);
#pragma unroll
    for (int a = 0; a < 3; ++a) {
      const uint64_t w = a == 0 ? w0 : (a == 1 ? w1 : w2);
      if (!((w >> (p & 63)) & 1ull)) continue;
      const int64_t vid = prefix[a * nwa + m] + __popcll(w & low);
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
  const int64_t P = R + 1, NP = P * P * P, NC = (int64_t)R * R * R;
  SurfaceWs w{};
  w.nwa = (NP + 63) / 64;
  w.nwords = 3 * w.nwa;
  w.nwb = (w.nwords + SF_WPB - 1) / SF_WPB;
  const int64_t pieces = (int64_t)R * R * ((R + 63) / 64);
  w.ncb = (pieces + SF_PPB - 1) / SF_PPB;
  (void)NC;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) / 256 * 256;
    return o;
  };
  w.off_words = take(8 * w.nwords);
  w.off_ins = take(8 * (w.nwa + 1));
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
  uint64_t* ins = reinterpret_cast<uint64_t*>(ws + w.off_ins);
  int32_t* prefix = reinterpret_cast<int32_t*>(ws + w.off_prefix);
  int64_t* wpart = reinterpret_cast<int64_t*>(ws + w.off_wpart);
  int64_t* cpart = reinterpret_cast<int64_t*>(ws + w.off_cpart);
  const int64_t cus = dev_info().cus;
  const int nwa = (int)w.nwa, nwords = (int)w.nwords, nwb = (int)w.nwb, ncb = (int)w.ncb;
  hipLaunchKernelGGL(sf_edges_kernel, dim3(grid_blocks(w.nwa, SF_NT / 64, 64 * cus)), dim3(SF_NT), 0, s, vol, R,
                     mask, words, ins, nwa);
  hipLaunchKernelGGL(sf_word_sums_kernel, dim3(nwb), dim3(SF_NT), 0, s, words, nwords, wpart);
  hipLaunchKernelGGL(sf_scan_parts_kernel, dim3(1), dim3(SF_NT), 0, s, wpart, nwb, counts);
  hipLaunchKernelGGL(sf_word_prefix_kernel, dim3(nwb), dim3(SF_NT), 0, s, words, nwords, wpart, prefix);
  hipLaunchKernelGGL(sf_cell_sums_kernel, dim3(ncb), dim3(SF_NT), 0, s, ins, R, mask, cpart);
  hipLaunchKernelGGL(sf_scan_parts_kernel, dim3(1), dim3(SF_NT), 0, s, cpart, ncb, counts + 1);
  hipLaunchKernelGGL(sf_triangles_kernel, dim3(ncb), dim3(SF_NT), 0, s, ins, R, mask, words, prefix, nwa, cpart, tris,
                     max_tris);
  hipLaunchKernelGGL(sf_vertices_kernel, dim3(grid_blocks(64 * w.nwa, SF_NT, 64 * cus)), dim3(SF_NT), 0, s, vol, R,
                     words, prefix, nwa, verts, max_verts, vert_edges);
  return hipGetLastError();
}

}  // namespace vdm
