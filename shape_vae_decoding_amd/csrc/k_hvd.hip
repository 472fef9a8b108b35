// Hierarchical Volume Decoding: the memory-bound stages between two decodes.
// FlashVDM summary page, section 4.1 item 1 (decode a coarse volume, find the
// voxels the surface crosses by a sign change between neighbouring samples,
// refine only those; key details: a truncated-SDF band keeps thin parts and one
// dilation guards against discretisation misses); techwalker article, part 2
// (wholly inside / outside regions keep their label without detailed queries).
//
// Bit masks use a blocked layout: point or cell (i, j, k) of a level with P
// points per axis lives in 64-bit word ((bi*NB + bj)*NB + bk)*8 + i%8, bit
// (j%8)*8 + k%8, with b = index/8 and NB = ceil(P/8). One 8x8x8 block is 8
// words; a workgroup of 8 waves covers one block with one lane per point
// (wave = i%8, lane = (j%8)*8 + k%8), so a wave ballot produces one word.
// Query lists are emitted in this same block order (blocked key order).
#include "vdm_device.hpp"
#include "vdm_hvd.hpp"

namespace vdm {

__device__ __forceinline__ bool mask_bit(const uint64_t* m, int NB, int i, int j, int k) {
  const int64_t w = ((int64_t)((i >> 3) * NB + (j >> 3)) * NB + (k >> 3)) * 8 + (i & 7);
  return (m[w] >> (((j & 7) << 3) | (k & 7))) & 1ull;
}

__device__ __forceinline__ int64_t block_sum_i64(int64_t v, int64_t* red, int tid, int nt) {
  // workgroup sum in fixed order (LDS of nt/64 slots)
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor((long long)v, o);
  if ((tid & 63) == 0) red[tid >> 6] = v;
  __syncthreads();
  int64_t s = 0;
  if (tid == 0)
    for (int w = 0; w < nt / 64; ++w) s += red[w];
  __syncthreads();
  return s;
}

__global__ void zero_u64_kernel(BP<uint64_t> pb, int64_t n) {
  uint64_t* p = pb.at();
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0ull;
}

hipError_t launch_zero_b(BP<void> p, size_t bytes, int B, hipStream_t s) {
  const int64_t n = (int64_t)(bytes / 8);
  if (n <= 0) return hipSuccess;
  int64_t g = (n + 255) / 256;
  if (g > 65536) g = 65536;
  hipLaunchKernelGGL(zero_u64_kernel, dim3((unsigned)g, (unsigned)B), dim3(256), 0, s,
                     BP<uint64_t>{(uint64_t*)p.p, p.stride}, n);
  return hipGetLastError();
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) { return launch_zero_b(bp(p), bytes, 1, s); }

__global__ void stats_init_kernel(BP<int64_t> sb, int levels, int R0) {
  int64_t* stats = sb.at();
  const int i = threadIdx.x;
  if (i < levels * VDM_STAT_FIELDS) stats[i] = (i % VDM_STAT_FIELDS) == VDM_STAT_R ? (int64_t)R0 << (i / VDM_STAT_FIELDS) : 0;
}

hipError_t launch_stats_init(BP<int64_t> stats, int levels, int R0, int B, hipStream_t s) {
  hipLaunchKernelGGL(stats_init_kernel, dim3(1, (unsigned)B), dim3(VDM_MAX_LEVELS * VDM_STAT_FIELDS), 0, s, stats,
                     levels, R0);
  return hipGetLastError();
}

// ------------------------------------------------------------------ counters
// Per-workgroup counts are added to STAT_SLOTS spread-out partial counters (slot =
// workgroup id mod STAT_SLOTS, 64 bytes apart) rather than to one address that
// every workgroup would contend for; fold_kernel then adds the slots into the
// level's stats and clears them for the next use.
constexpr int STAT_SLOTS = 256;

__global__ __launch_bounds__(STAT_SLOTS) void fold_kernel(BP<int64_t> pb, int f0, int nf, BP<int64_t> d0,
                                                          BP<int64_t> d1) {
  __shared__ int64_t red[STAT_SLOTS / 64];
  int64_t* part = pb.at();
  int64_t* dst0 = d0.at();
  int64_t* dst1 = d1.at();
  const int t = threadIdx.x;
  for (int f = 0; f < nf; ++f) {
    const int64_t v = part[t * 8 + f0 + f];
    part[t * 8 + f0 + f] = 0;
    const int64_t sum = block_sum_i64(v, red, t, STAT_SLOTS);
    if (t == 0) *(f == 0 ? dst0 : dst1) += sum;
  }
}

static hipError_t launch_fold(BP<int64_t> part, int f0, int nf, BP<int64_t> dst0, BP<int64_t> dst1, int B,
                              hipStream_t s) {
  hipLaunchKernelGGL(fold_kernel, dim3(1, (unsigned)B), dim3(STAT_SLOTS), 0, s, part, f0, nf, dst0, dst1);
  return hipGetLastError();
}

// ------------------------------------------------------------------ cell test
// Cell (i, j, k) of level L (R cells per axis) is tested when all 8 corners were
// computed: every cell at level 0, the children of kept parents afterwards
// (kept_prev = the previous level's kept cells; null at level 0). A tested cell
// is active when its corner values include s < 0 and s >= 0, or min |s| < tau.
// One wave tests one 8x8x8 cell block: lane (jj, kk) holds the 9 x 2 x 2 corner
// values of its column of cells (i = 8bi .. 8bi+7), 36 loads in flight at once
// (indexes clamped into the volume: clamped points belong only to cells that are
// not tested), and each of the 8 cell rows gives one ballot word. Level 0 has one
// wave per cell block. Above it one wave takes the 2x2x2 child blocks of one parent
// block: the parent block's 8 words (scalar loads) decide which child blocks hold a
// child of a kept parent, the others only get their zero words, and a cell's parent
// bit comes from the same registers. (Loading two tested blocks at a time measured
// slower: the registers it takes cost more occupancy than the overlap gains.)
__device__ __forceinline__ bool child_block(int NB, int gi, int gj, int gk, int c, int& bi, int& bj, int& bk) {
  bi = 2 * gi + (c >> 2);
  bj = 2 * gj + ((c >> 1) & 1);
  bk = 2 * gk + (c & 1);
  return bi < NB && bj < NB && bk < NB;
}

// Corner values of the column of cells (i = 8bi .. 8bi+7, j = 8bj + lane/8,
// k = 8bk + lane%8): v[a][e] = point (8bi + a, j + e/2, k + e%2), clamped into the volume.
__device__ __forceinline__ void load_cell_block(const float* __restrict__ vol, int R, int bi, int bj, int bk, int lane,
                                                float (&v)[9][4]) {
  const int64_t P = R + 1;
  const int J = 8 * bj + (lane >> 3), K = 8 * bk + (lane & 7);
  const int64_t Ja = min(J, R) * P, Jb = min(J + 1, R) * P;
  const int Ka = min(K, R), Kb = min(K + 1, R);
#pragma unroll
  for (int a = 0; a < 9; ++a) {
    const float* row = vol + (int64_t)min(8 * bi + a, R) * P * P;
    v[a][0] = row[Ja + Ka];
    v[a][1] = row[Ja + Kb];
    v[a][2] = row[Jb + Ka];
    v[a][3] = row[Jb + Kb];
  }
}

// Test the block's 512 cells, write its 8 active words, add to the wave's counts.
// SPARSE: the parent bit of cell row ii is pw[r0 + ii/2] >> psh.
template <bool SPARSE>
__device__ __forceinline__ void test_cell_block(const float (&v)[9][4], int R, int NB, int bi, int bj, int bk,
                                                int lane, const uint64_t (&pw)[8], int r0, int psh, float tau,
                                                uint64_t* __restrict__ active, int& nt, int& na) {
  const bool in_jk = 8 * bj + (lane >> 3) < R && 8 * bk + (lane & 7) < R;
  uint64_t mine = 0;
#pragma unroll
  for (int ii = 0; ii < 8; ++ii) {
    bool tested = in_jk && 8 * bi + ii < R;
    if (SPARSE) tested = tested && ((pw[r0 + (ii >> 1)] >> psh) & 1ull);
    bool neg = false, nonneg = false;
    float mn = __builtin_inff();
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float sv = v[ii + a][e];
        neg |= sv < 0.f;
        nonneg |= sv >= 0.f;
        mn = fminf(mn, fabsf(sv));
      }
    const bool act = tested && ((neg && nonneg) || mn < tau);
    const uint64_t tw = __ballot(tested), aw = __ballot(act);
    nt += __popcll(tw);
    na += __popcll(aw);
    if (lane == ii) mine = aw;
  }
  if (lane < 8) active[(((int64_t)bi * NB + bj) * NB + bk) * 8 + lane] = mine;
}

template <bool SPARSE>
__global__ __launch_bounds__(256) void cell_test_kernel(BP<const float> vb, int R, int NB, BP<const uint64_t> kb,
                                                        int NBp, float tau, BP<uint64_t> ab, BP<int64_t> pb,
                                                        int nunits) {
  const float* __restrict__ vol = vb.at();
  const uint64_t* __restrict__ kept_prev = kb.at();
  uint64_t* __restrict__ active = ab.at();
  int64_t* part = pb.at();
  const int lane = threadIdx.x & 63;
  const int u = __builtin_amdgcn_readfirstlane((int)blockIdx.x * 4 + (int)(threadIdx.x >> 6));
  if (u >= nunits) return;
  int nt = 0, na = 0;
  uint64_t pw[8];
  if (!SPARSE) {  // unit = one cell block
#pragma unroll
    for (int r = 0; r < 8; ++r) pw[r] = ~0ull;
    const int bi = u / (NB * NB), bj = (u / NB) % NB, bk = u % NB;
    float v[9][4];
    load_cell_block(vol, R, bi, bj, bk, lane, v);
    test_cell_block<false>(v, R, NB, bi, bj, bk, lane, pw, 0, 0, tau, active, nt, na);
  } else {  // unit = the 2x2x2 child blocks of parent block u
    const int NG = (NB + 1) / 2;
    const int gi = u / (NG * NG), gj = (u / NG) % NG, gk = u % NG;
#pragma unroll
    for (int r = 0; r < 8; ++r) pw[r] = kept_prev[(((int64_t)gi * NBp + gj) * NBp + gk) * 8 + r];
    const int jj = lane >> 3, kk = lane & 7;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      int bi, bj, bk;
      if (!child_block(NB, gi, gj, gk, c, bi, bj, bk)) continue;
      // parents of child block c: rows 4(c>>2) .. +3 of the parent block, the 4x4
      // square (4bj .. 4bj+3) x (4bk .. 4bk+3) of each row's word
      const int r0 = 4 * (c >> 2);
      const uint64_t sq = 0x0f0f0f0full << (((c >> 1) & 1) * 32 + (c & 1) * 4);
      if (((pw[r0] | pw[r0 + 1] | pw[r0 + 2] | pw[r0 + 3]) & sq) == 0ull) {
        if (lane < 8) active[(((int64_t)bi * NB + bj) * NB + bk) * 8 + lane] = 0ull;
        continue;
      }
      // parent of cell (i, j, k) = (i/2, j/2, k/2): row r0 + ii/2, bit
      // (4((c>>1)&1) + jj/2) * 8 + 4(c&1) + kk/2
      const int psh = (4 * ((c >> 1) & 1) + (jj >> 1)) * 8 + 4 * (c & 1) + (kk >> 1);
      float v[9][4];
      load_cell_block(vol, R, bi, bj, bk, lane, v);
      test_cell_block<true>(v, R, NB, bi, bj, bk, lane, pw, r0, psh, tau, active, nt, na);
    }
  }
  if (lane == 0 && (nt | na)) {
    int64_t* slot = part + (u % STAT_SLOTS) * 8;
    if (nt) atomicAdd((unsigned long long*)slot, (unsigned long long)nt);
    if (na) atomicAdd((unsigned long long*)(slot + 1), (unsigned long long)na);
  }
}

hipError_t launch_cell_test(BP<const float> vol, int R, BP<const uint64_t> kept_prev, float tau, BP<uint64_t> active,
                            BP<int64_t> part, BP<int64_t> stat_tested, BP<int64_t> stat_active, int B, hipStream_t s) {
  const int NB = nblocks8(R + 1), NBp = nblocks8(R / 2 + 1), NG = (NB + 1) / 2;
  const int nunits = kept_prev.p ? NG * NG * NG : NB * NB * NB;
  const dim3 grid((unsigned)((nunits + 3) / 4), (unsigned)B);
  if (kept_prev.p)
    hipLaunchKernelGGL(cell_test_kernel<true>, grid, dim3(256), 0, s, vol, R, NB, kept_prev, NBp, tau, active, part,
                       nunits);
  else
    hipLaunchKernelGGL(cell_test_kernel<false>, grid, dim3(256), 0, s, vol, R, NB, kept_prev, NBp, tau, active,
                       part, nunits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_fold(part, 0, 2, stat_tested, stat_active, B, s);
}

// ------------------------------------------------------------------ dilation
// One thread per word (8 consecutive lanes: the 8 rows of one block, so every
// load of a wave reads whole 64-byte blocks): OR over the 3x3x3 neighbourhood,
// separably along k (bit shifts inside each 8-bit row), j (shifts by 8) and i
// (neighbouring rows), with neighbour blocks supplying the halo. Cells outside
// [0, R)^3 stay clear.
__device__ __forceinline__ uint64_t dil_k(uint64_t w, uint64_t wl, uint64_t wr) {
  const uint64_t C0 = 0x0101010101010101ull, C7 = 0x8080808080808080ull;
  return w | ((w << 1) & ~C0) | ((wl >> 7) & C0) | ((w >> 1) & ~C7) | ((wr << 7) & C7);
}
__device__ __forceinline__ uint64_t dil_j(uint64_t t, uint64_t td, uint64_t tu) {
  return t | (t << 8) | (td >> 56) | (t >> 8) | (tu << 56);
}

// Bits of the 8x8 (j, k) cells of block (bj, bk) that lie inside [0, lim)^2.
__device__ __forceinline__ uint64_t inside_jk(int lim, int bj, int bk) {
  const int nj = min(max(lim - 8 * bj, 0), 8), nk = min(max(lim - 8 * bk, 0), 8);
  const uint64_t rows = nj >= 8 ? ~0ull : ((1ull << (8 * nj)) - 1ull);
  return (nk >= 8 ? ~0ull : ((1ull << nk) - 1ull) * 0x0101010101010101ull) & rows;
}

// The 8 words of a block as four 16-byte stores (block words are 64-byte aligned).
__device__ __forceinline__ void store_block(uint64_t* __restrict__ dst, const uint64_t (&w)[8]) {
#pragma unroll
  for (int h = 0; h < 4; ++h)
    reinterpret_cast<uint4*>(dst)[h] =
        make_uint4((uint32_t)w[2 * h], (uint32_t)(w[2 * h] >> 32), (uint32_t)w[2 * h + 1], (uint32_t)(w[2 * h + 1] >> 32));
}

__global__ __launch_bounds__(256) void dilate_kernel(BP<const uint64_t> ib, BP<uint64_t> ob, int R, int NB, int identity,
                                                     BP<int64_t> pb) {
  __shared__ int64_t red[4];
  const uint64_t* __restrict__ in = ib.at();
  uint64_t* __restrict__ out = ob.at();
  int64_t* part = pb.p ? pb.at() : nullptr;
  const int w = (int)blockIdx.x * 256 + (int)threadIdx.x;  // word; NB^3 * 8 < 2^31 (R <= 1200)
  uint64_t res = 0;
  if (w < NB * NB * NB * 8) {
    const int b = w >> 3, ii = w & 7;
    const int bi = b / (NB * NB), r2 = b - bi * NB * NB, bj = r2 / NB, bk = r2 - bj * NB;
    const int i = 8 * bi + ii;
    if (i < R && identity) {
      res = in[w];
    } else if (i < R) {
#pragma unroll
      for (int di = -1; di <= 1; ++di) {
        const int i2 = i + di;
        if (i2 < 0 || i2 >= R) continue;
        const int64_t base = (int64_t)(i2 >> 3) * NB;
        uint64_t W[3][3];
#pragma unroll
        for (int a = 0; a < 3; ++a)
#pragma unroll
          for (int c = 0; c < 3; ++c) {
            const int bj2 = bj + a - 1, bk2 = bk + c - 1;
            W[a][c] = (bj2 >= 0 && bj2 < NB && bk2 >= 0 && bk2 < NB) ? in[((base + bj2) * NB + bk2) * 8 + (i2 & 7)] : 0ull;
          }
        res |= dil_j(dil_k(W[1][1], W[1][0], W[1][2]), dil_k(W[0][1], W[0][0], W[0][2]), dil_k(W[2][1], W[2][0], W[2][2]));
      }
    }
    res &= i < R ? inside_jk(R, bj, bk) : 0ull;  // clip to cells inside the grid
    out[w] = res;
  }
  if (part) {
    const int64_t n = block_sum_i64(__popcll(res), red, threadIdx.x, 256);
    if (threadIdx.x == 0 && n) atomicAdd((unsigned long long*)(part + (blockIdx.x % STAT_SLOTS) * 8 + 2), (unsigned long long)n);
  }
}

hipError_t launch_dilate(BP<const uint64_t> in, BP<uint64_t> out, int R, int identity, BP<int64_t> part,
                         BP<int64_t> stat, int B, hipStream_t s) {
  const int NB = nblocks8(R + 1);
  const int64_t nw = (int64_t)NB * NB * NB * 8;
  hipLaunchKernelGGL(dilate_kernel, dim3((unsigned)((nw + 255) / 256), (unsigned)B), dim3(256), 0, s, in, out, R, NB,
                     identity, stat.p ? part : BP<int64_t>{nullptr, 0});
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !stat.p) return e;
  return launch_fold(part, 2, 1, stat, stat, B, s);
}

// ------------------------------------------------------------------ child marking
// Point (I, J, K) of level L+1 (Rn = 2R cells) is a candidate when it is a corner
// of a child of a kept level-L cell: per axis, even X has parents X/2 - 1 and X/2,
// odd X has parent (X-1)/2. It is new when it was not computed before: a point
// with all-even indices was computed iff its level-L point (I/2, J/2, K/2) was
// (every point at level 0). all_new: every in-range point is new (level 0 list).
//
// Bit-parallel, one thread per 8x8x8 point block (bi, bj, bk). Its points have
// parent cells in rows a = 4bi-1 .. 4bi+3, and in each row the 5x5 window
// c = 4bj-1 .. 4bj+3, d = 4bk-1 .. 4bk+3 (up to 4 words: the main quadrant and the
// j-, k- and corner halos). Each row's window, packed as 5 bytes of 5 bits, is
// "upsampled" by the parent rule along k (bits) and j (bytes) with spread
// operations on the whole word; output row I takes the rows of its parents.

// The low 4 bits of every byte to bits 0, 2, 4, 6 of that byte.
__device__ __forceinline__ uint64_t spread_bits(uint64_t t) {
  t = (t | (t << 2)) & 0x3333333333333333ull;
  return (t | (t << 1)) & 0x5555555555555555ull;
}
// The low 4 bytes of a word to bytes 0, 2, 4, 6.
__device__ __forceinline__ uint64_t spread_bytes(uint64_t t) {
  t = (t | (t << 16)) & 0x0000ffff0000ffffull;
  return (t | (t << 8)) & 0x00ff00ff00ff00ffull;
}
// 5x5 window X (byte r = parent row 4bj-1+r, bit c = parent column 4bk-1+c) to
// the 8x8 candidate word: point 2m+1 has parent m+1 of the window, point 2m
// parents m and m+1, along each axis.
__device__ __forceinline__ uint64_t upsample_window(uint64_t X) {
  const uint64_t E = spread_bits((X >> 1) & 0x0f0f0f0f0full);
  const uint64_t Y = spread_bits(X & 0x0f0f0f0f0full) | E | (E << 1);
  const uint64_t H = spread_bytes((Y >> 8) & 0xffffffffull);
  return spread_bytes(Y & 0xffffffffull) | H | (H << 8);
}

// Candidate word of point block (., bj, bk) of level L+1 from kept parent row a
// (kept: level-L cell mask, R cells, NB blocks; bits outside [0, R)^3 are clear).
__device__ __forceinline__ uint64_t cand_row(const uint64_t* __restrict__ kept, int NB, int R, int a, int bj, int bk) {
  if (a < 0 || a >= R) return 0ull;
  const int64_t rb = (int64_t)(a >> 3) * NB;
  const int Cm = bj >> 1, Dm = bk >> 1, jo = bj & 1, ko = bk & 1;
  auto ld = [&](int C, int Dd) { return kept[((rb + C) * NB + Dd) * 8 + (a & 7)]; };
  const uint64_t Wm = ld(Cm, Dm);
  const uint64_t Wj = jo ? Wm : (bj > 0 ? ld(Cm - 1, Dm) : 0ull);  // holds parent row 4bj-1
  const uint64_t Wk = ko ? Wm : (bk > 0 ? ld(Cm, Dm - 1) : 0ull);  // holds parent column 4bk-1
  const uint64_t Wc = jo ? Wk : (ko ? Wj : ((bj > 0 && bk > 0) ? ld(Cm - 1, Dm - 1) : 0ull));
  const int hr = jo ? 3 : 7, hc = ko ? 3 : 7;  // (4bj-1) & 7 and (4bk-1) & 7
  uint64_t X = ((Wm >> (32 * jo + 4 * ko)) & 0x0f0f0f0full) << 9;
  X |= ((Wk >> (32 * jo + hc)) & 0x01010101ull) << 8;
  X |= ((Wj >> (8 * hr + 4 * ko)) & 0xfull) << 1;
  X |= (Wc >> (8 * hr + hc)) & 1ull;
  return upsample_window(X);
}

__global__ __launch_bounds__(256) void mark_kernel(BP<const uint64_t> kb, int R, BP<const uint64_t> cpb, int all_new,
                                                   int Rn, BP<uint64_t> nmb, BP<uint64_t> cnb, BP<int32_t> cb) {
  const uint64_t* __restrict__ kept = kb.p ? kb.at() : nullptr;
  const uint64_t* __restrict__ comp_prev = cpb.p ? cpb.at() : nullptr;
  uint64_t* __restrict__ newmask = nmb.at();
  uint64_t* __restrict__ comp_next = cnb.p ? cnb.at() : nullptr;
  int32_t* __restrict__ counts = cb.at();
  const int NBn = nblocks8(Rn + 1), NB = nblocks8(R + 1);
  const int b = (int)blockIdx.x * 256 + (int)threadIdx.x;
  if (b >= NBn * NBn * NBn) return;
  const int bi = b / (NBn * NBn), r2 = b - bi * NBn * NBn, bj = r2 / NBn, bk = r2 - bj * NBn;
  const uint64_t inr = inside_jk(Rn + 1, bj, bk);  // points inside [0, Rn]^2
  uint64_t wn[8], wc[8];
  if (all_new) {
#pragma unroll
    for (int ii = 0; ii < 8; ++ii) wn[ii] = wc[ii] = 8 * bi + ii <= Rn ? inr : 0ull;
  } else {
    uint64_t C[5];
#pragma unroll
    for (int r = 0; r < 5; ++r) C[r] = cand_row(kept, NB, R, 4 * bi - 1 + r, bj, bk);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      // even row I = 8bi+2m: parents 4bi+m-1 and 4bi+m; computed before where all-even
      const int I = 8 * bi + 2 * m;
      const uint64_t in_e = I <= Rn ? inr : 0ull;
      uint64_t wp = 0ull;
      if (I <= Rn) {
        if (comp_prev) {
          const int i2 = I >> 1;
          const uint64_t pw = comp_prev[(((int64_t)(i2 >> 3) * NB + (bj >> 1)) * NB + (bk >> 1)) * 8 + (i2 & 7)];
          wp = spread_bytes(spread_bits((pw >> (32 * (bj & 1) + 4 * (bk & 1))) & 0x0f0f0f0full));
        } else {
          wp = 0x0055005500550055ull;
        }
        wp &= in_e;
      }
      wn[2 * m] = (C[m] | C[m + 1]) & ~wp & in_e;
      wc[2 * m] = wn[2 * m] | wp;
      // odd row I + 1: parent 4bi+m
      wn[2 * m + 1] = wc[2 * m + 1] = C[m + 1] & (I + 1 <= Rn ? inr : 0ull);
    }
  }
  int c = 0;
#pragma unroll
  for (int ii = 0; ii < 8; ++ii) c += __popcll(wn[ii]);
  store_block(newmask + (int64_t)b * 8, wn);
  if (comp_next) store_block(comp_next + (int64_t)b * 8, wc);
  counts[b] = c;
}

hipError_t launch_mark(BP<const uint64_t> kept, int R, BP<const uint64_t> comp_prev, int all_new, int Rn,
                       BP<uint64_t> newmask, BP<uint64_t> comp_next, BP<int32_t> counts, int B, hipStream_t s) {
  const int NBn = nblocks8(Rn + 1);
  const int64_t nb3 = (int64_t)NBn * NBn * NBn;
  hipLaunchKernelGGL(mark_kernel, dim3((unsigned)((nb3 + 255) / 256), (unsigned)B), dim3(256), 0, s, kept, R,
                     comp_prev, all_new, Rn, newmask, comp_next, counts);
  return hipGetLastError();
}

// ------------------------------------------------------------------ scan of per-block counts
// For each block: queries q = counts[b], work items ceil(q / bq), occupied (q > 0).
// Exclusive prefix sums give each block's offsets in the list, the item array and
// the occupied-block array (which the last pass fills); totals go to tot[0..2]
// and to the level's stats.
constexpr int SCAN_NT = 256;
constexpr int SCAN_PER = 8;
constexpr int SCAN_CHUNK = SCAN_NT * SCAN_PER;

__device__ __forceinline__ int4 tuple_of(int c, int bq) { return make_int4(c, (c + bq - 1) / bq, c > 0, 0); }
__device__ __forceinline__ int4 add4(int4 a, int4 b) { return make_int4(a.x + b.x, a.y + b.y, a.z + b.z, 0); }

__device__ int4 block_excl_scan(int4 v, int4* sh, int tid, int4* total) {
  sh[tid] = v;
  __syncthreads();
  for (int o = 1; o < SCAN_NT; o <<= 1) {
    int4 u = tid >= o ? sh[tid - o] : make_int4(0, 0, 0, 0);
    __syncthreads();
    sh[tid] = add4(sh[tid], u);
    __syncthreads();
  }
  const int4 incl = sh[tid];
  *total = sh[SCAN_NT - 1];
  __syncthreads();
  return make_int4(incl.x - v.x, incl.y - v.y, incl.z - v.z, 0);
}

__global__ __launch_bounds__(SCAN_NT) void scan_reduce_kernel(BP<const int32_t> cb, int64_t n, int bq, BP<int4> pb) {
  __shared__ int4 sh[SCAN_NT];
  const int32_t* counts = cb.at();
  int4* partial = pb.at();
  const int64_t base = (int64_t)blockIdx.x * SCAN_CHUNK + threadIdx.x * SCAN_PER;
  int4 s = make_int4(0, 0, 0, 0);
  for (int e = 0; e < SCAN_PER; ++e)
    if (base + e < n) s = add4(s, tuple_of(counts[base + e], bq));
  int4 tot;
  block_excl_scan(s, sh, threadIdx.x, &tot);
  if (threadIdx.x == 0) partial[blockIdx.x] = tot;
}

__global__ __launch_bounds__(SCAN_NT) void scan_top_kernel(BP<int4> pb, int np, BP<int32_t> tb, BP<int64_t> sb) {
  __shared__ int4 sh[SCAN_NT];
  int4* partial = pb.at();
  int32_t* tot = tb.at();
  int64_t* stats_level = sb.p ? sb.at() : nullptr;
  int4 carry = make_int4(0, 0, 0, 0);
  for (int base = 0; base < np; base += SCAN_NT) {
    const int i = base + threadIdx.x;
    const int4 v = i < np ? partial[i] : make_int4(0, 0, 0, 0);
    int4 t;
    const int4 ex = block_excl_scan(v, sh, threadIdx.x, &t);
    if (i < np) partial[i] = add4(ex, carry);
    carry = add4(carry, t);
  }
  if (threadIdx.x == 0) {
    tot[0] = carry.x;
    tot[1] = carry.y;
    tot[2] = carry.z;
    if (stats_level) {
      stats_level[VDM_STAT_QUERIES] = carry.x;
      stats_level[VDM_STAT_ITEMS] = carry.y;
      stats_level[VDM_STAT_BLOCKS] = carry.z;
    }
  }
}

__global__ __launch_bounds__(SCAN_NT) void scan_apply_kernel(BP<const int32_t> cb, int64_t n, int bq,
                                                             BP<const int4> pb, BP<int4> ob, BP<int32_t> occb) {
  __shared__ int4 sh[SCAN_NT];
  const int32_t* counts = cb.at();
  const int4* partial = pb.at();
  int4* offs = ob.at();
  int32_t* occ = occb.at();
  const int64_t base = (int64_t)blockIdx.x * SCAN_CHUNK + threadIdx.x * SCAN_PER;
  int4 v[SCAN_PER];
  int4 s = make_int4(0, 0, 0, 0);
  for (int e = 0; e < SCAN_PER; ++e) {
    v[e] = base + e < n ? tuple_of(counts[base + e], bq) : make_int4(0, 0, 0, 0);
    s = add4(s, v[e]);
  }
  int4 tot;
  int4 run = add4(block_excl_scan(s, sh, threadIdx.x, &tot), partial[blockIdx.x]);
  for (int e = 0; e < SCAN_PER; ++e) {
    if (base + e < n) {
      offs[base + e] = run;
      if (v[e].z && VDM_BOUND(run.z < n, BC_SCAN_OCC)) occ[run.z] = (int32_t)(base + e);  // occupied blocks in block order
    }
    run = add4(run, v[e]);
  }
}

hipError_t launch_scan(BP<const int32_t> counts, int64_t n, int bq, BP<int4> partial, BP<int4> offs, BP<int32_t> occ,
                       BP<int32_t> tot, BP<int64_t> stats_level, int B, hipStream_t s) {
  const int np = (int)((n + SCAN_CHUNK - 1) / SCAN_CHUNK);
  hipLaunchKernelGGL(scan_reduce_kernel, dim3(np, (unsigned)B), dim3(SCAN_NT), 0, s, counts, n, bq, partial);
  hipLaunchKernelGGL(scan_top_kernel, dim3(1, (unsigned)B), dim3(SCAN_NT), 0, s, partial, np, tot, stats_level);
  hipLaunchKernelGGL(scan_apply_kernel, dim3(np, (unsigned)B), dim3(SCAN_NT), 0, s, counts, n, bq,
                     BP<const int4>{partial.p, partial.stride}, offs, occ);
  return hipGetLastError();
}

// ------------------------------------------------------------------ emit lists
// One wave per occupied block (occ[0 .. tot[2]), grid-strided): the block writes
// its new points (row-major linear indices, in-block row-major order) at its list
// offset and its work items (query chunks of at most bq, all attending to
// occupied-block row offs.z).
constexpr int EMIT_NT = 256;

__global__ __launch_bounds__(EMIT_NT) void emit_kernel(BP<const uint64_t> nmb, BP<const int32_t> cb,
                                                       BP<const int4> ob, BP<const int32_t> occb,
                                                       BP<const int32_t> tb, int Rn, int bq, BP<int32_t> lb,
                                                       BP<Item> ib, int64_t list_cap, int64_t item_cap) {
  const uint64_t* __restrict__ newmask = nmb.at();
  const int32_t* __restrict__ counts = cb.at();
  const int4* __restrict__ offs = ob.at();
  const int32_t* __restrict__ occ = occb.at();
  const int32_t* __restrict__ tot = tb.at();
  int32_t* __restrict__ list = lb.at();
  Item* __restrict__ items = ib.at();
  const int NB = nblocks8(Rn + 1);
  const int64_t P = Rn + 1;
  const int lane = threadIdx.x & 63;
  const int nocc = tot[2];
  const int wpb = EMIT_NT / 64;
  for (int o = blockIdx.x * wpb + (threadIdx.x >> 6); o < nocc; o += gridDim.x * wpb) {
    const int64_t b = occ[o];
    const int c = counts[b];
    const int4 of = offs[b];
    const int bi = (int)(b / ((int64_t)NB * NB)), bj = (int)((b / NB) % NB), bk = (int)(b % NB);
    const int J = 8 * bj + (lane >> 3), K = 8 * bk + (lane & 7);
    int before = 0;
#pragma unroll
    for (int ii = 0; ii < 8; ++ii) {
      const uint64_t w = newmask[b * 8 + ii];
      if ((w >> lane) & 1ull) {
        const int rank = before + __popcll(w & ((1ull << lane) - 1ull));
        if (VDM_BOUND((int64_t)of.x + rank < list_cap, BC_EMIT_LIST))
          list[of.x + rank] = (int32_t)(((int64_t)(8 * bi + ii) * P + J) * P + K);
      }
      before += __popcll(w);
    }
    const int nchunks = (c + bq - 1) / bq;
    for (int ch = lane; ch < nchunks; ch += 64) {
      const int q0 = of.x + ch * bq;
      if (VDM_BOUND((int64_t)of.y + ch < item_cap, BC_EMIT_ITEM)) items[of.y + ch] = Item{q0, min(q0 + bq, of.x + c), of.z, 0};
    }
  }
}

hipError_t launch_emit(BP<const uint64_t> newmask, BP<const int32_t> counts, BP<const int4> offs,
                       BP<const int32_t> occ, BP<const int32_t> tot, int Rn, int bq, BP<int32_t> list,
                       int64_t list_cap, BP<Item> items, int64_t item_cap, int B, hipStream_t s) {
  const int NB = nblocks8(Rn + 1);
  const int64_t nb3 = (int64_t)NB * NB * NB;
  int64_t g = (nb3 + EMIT_NT / 64 - 1) / (EMIT_NT / 64);
  const int64_t cap = ((int64_t)dev_info().cus * 8 + B - 1) / B;
  if (g > cap) g = cap;
  if (g < 1) g = 1;
  hipLaunchKernelGGL(emit_kernel, dim3((unsigned)g, (unsigned)B), dim3(EMIT_NT), 0, s, newmask, counts, offs, occ, tot,
                     Rn, bq, list, items, list_cap, item_cap);
  return hipGetLastError();
}

// ------------------------------------------------------------------ nearest-ancestor fill
// vol_next[I][J][K] = vol_prev[I/2][J/2][K/2] (integer division) for every point.
// The output is one flat array cut into groups of 4 consecutive values, aligned
// so that each group is one 16-byte store (the few values before the first
// aligned address and after the last whole group are written one by one). A
// workgroup writes FILL_U x 256 consecutive groups: all their source loads are
// issued before the first store. A group's (I, J, K) comes from a division (a
// double-precision reciprocal estimate, corrected exactly); inside one output row
// its 4 values need 2 or 3 consecutive source values. The output is not read back
// by this kernel and is larger than the caches, so it is stored non-temporally.
// Flat offsets are 32-bit: the finest volume holds at most 1201^3 < 2^32 points.
constexpr int FILL_NT = 256;
constexpr int FILL_U = 2;

struct Div32 {
  uint32_t d;
  double inv;
};

// floor(n / d): n * (1/d) in double is within one of the quotient for n < 2^32,
// then one exact correction.
__device__ __forceinline__ uint32_t div32(uint32_t n, const Div32& dv) {
  uint32_t q = (uint32_t)((double)n * dv.inv);
  const uint32_t qd = q * dv.d;
  if (qd > n)
    --q;
  else if (n - qd >= dv.d)
    ++q;
  return q;
}

__device__ __forceinline__ float fill_value(const float* __restrict__ prev, int Pp, int I, int J, int K) {
  return prev[((size_t)(I >> 1) * Pp + (J >> 1)) * Pp + (K >> 1)];
}

// the 4 values of the group that starts at flat offset o
__device__ __forceinline__ float4 fill_group(const float* __restrict__ prev, int Pp, int Pn, uint32_t o,
                                             const Div32& d2, const Div32& d1) {
  const uint32_t I = div32(o, d2), rem = o - I * d2.d;
  const uint32_t J = div32(rem, d1);
  uint32_t K = rem - J * d1.d;
  if (K + 3 < (uint32_t)Pn) {  // one output row: sources K/2 .. (K+3)/2
    const float* __restrict__ src = prev + ((size_t)(I >> 1) * Pp + (J >> 1)) * Pp + (K >> 1);
    const float a = src[0], b = src[1];
    if (K & 1) return make_float4(a, b, b, src[2]);
    return make_float4(a, a, b, b);
  }
  float v[4];
  uint32_t Ii = I, Jj = J;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    v[t] = fill_value(prev, Pp, (int)Ii, (int)Jj, (int)K);
    if (++K == (uint32_t)Pn) {
      K = 0;
      if (++Jj == (uint32_t)Pn) {
        Jj = 0;
        ++Ii;
      }
    }
  }
  return make_float4(v[0], v[1], v[2], v[3]);
}

typedef float fill_f4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(FILL_NT) void fill_kernel(BP<const float> pb, int Pp, BP<float> nb, int Pn, Div32 d2,
                                                       Div32 d1) {
  const float* __restrict__ prev = pb.at();
  float* __restrict__ next = nb.at();
  const uint32_t n = (uint32_t)Pn * Pn * Pn;
  // values before the first 16-byte aligned address, then whole groups of 4
  const uint32_t head = min((uint32_t)(((16 - ((uintptr_t)next & 15)) & 15) / 4), n);
  const uint32_t ngroups = (n - head) / 4;
  const uint32_t g0 = blockIdx.x * (FILL_NT * FILL_U) + threadIdx.x;
  float4 v[FILL_U];
#pragma unroll
  for (int u = 0; u < FILL_U; ++u) {
    const uint32_t g = g0 + u * FILL_NT;
    if (g < ngroups) v[u] = fill_group(prev, Pp, Pn, head + 4 * g, d2, d1);
  }
#pragma unroll
  for (int u = 0; u < FILL_U; ++u) {
    const uint32_t g = g0 + u * FILL_NT;
    if (g < ngroups) {
      const fill_f4 x = {v[u].x, v[u].y, v[u].z, v[u].w};
      __builtin_nontemporal_store(x, reinterpret_cast<fill_f4*>(next + head + 4 * g));
    }
  }
  if (blockIdx.x == 0 && threadIdx.x < head + ((n - head) & 3)) {
    const uint32_t o = threadIdx.x < head ? threadIdx.x : head + 4 * ngroups + (threadIdx.x - head);
    const uint32_t I = div32(o, d2), rem = o - I * d2.d;
    const uint32_t J = div32(rem, d1);
    next[o] = fill_value(prev, Pp, (int)I, (int)J, (int)(rem - J * d1.d));
  }
}

hipError_t launch_fill(BP<const float> prev, int Pp, BP<float> next, int Pn, int B, hipStream_t s) {
  if (Pn < 1 || Pn > 1201) return hipErrorInvalidValue;
  const int64_t n = (int64_t)Pn * Pn * Pn;
  const int64_t g = n / 4 / (FILL_NT * FILL_U) + 1;
  const Div32 d2{(uint32_t)(Pn * Pn), 1.0 / ((double)Pn * Pn)}, d1{(uint32_t)Pn, 1.0 / (double)Pn};
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)g, (unsigned)B), dim3(FILL_NT), 0, s, prev, Pp, next, Pn, d2, d1);
  return hipGetLastError();
}

// ------------------------------------------------------------------ tiles of a batch
// Exclusive prefix of the per-shape decode units of a batch (each shape's count is
// on the device, written by its scan): thread t sums the units of shapes
// t*S .. t*S+S-1 (S = ceil(B / 1024)), the 1024 sums are scanned in LDS, and each
// thread writes its shapes' prefixes; prefix[B] = every unit.
constexpr int PREFIX_NT = 1024;

__global__ __launch_bounds__(PREFIX_NT) void batch_prefix_kernel(const int32_t* __restrict__ cnt, int64_t stride, int B,
                                                                 int per, int64_t* __restrict__ prefix) {
  __shared__ int64_t part[PREFIX_NT];
  const int t = threadIdx.x;
  const int S = (B + PREFIX_NT - 1) / PREFIX_NT;
  auto units = [&](int b) -> int64_t {
    const int64_t c = cnt[(int64_t)b * stride];
    return c > 0 ? (c + per - 1) / per : 0;
  };
  int64_t sum = 0;
  for (int i = 0; i < S; ++i) {
    const int b = t * S + i;
    if (b < B) sum += units(b);
  }
  part[t] = sum;
  __syncthreads();
  for (int o = 1; o < PREFIX_NT; o <<= 1) {  // inclusive scan of the thread sums
    const int64_t v = t >= o ? part[t - o] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int64_t run = t > 0 ? part[t - 1] : 0;
  for (int i = 0; i < S; ++i) {
    const int b = t * S + i;
    if (b < B) {
      prefix[b] = run;
      run += units(b);
    }
  }
  if (t == PREFIX_NT - 1) prefix[B] = part[PREFIX_NT - 1];
}

hipError_t launch_batch_prefix(const int32_t* cnt, int64_t stride, int B, int per, int64_t* prefix, hipStream_t s) {
  if (B < 1 || B > 4096 || per < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(batch_prefix_kernel, dim3(1), dim3(PREFIX_NT), 0, s, cnt, stride, B, per, prefix);
  return hipGetLastError();
}

// ------------------------------------------------------------------ inspection export
// Row-major byte mask of an n^3 region of a blocked bit mask.
__global__ void bits_to_bytes_kernel(const uint64_t* __restrict__ m, int n, int NB, uint8_t* __restrict__ out) {
  const int64_t tot = (int64_t)n * n * n;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < tot; t += (int64_t)gridDim.x * blockDim.x) {
    const int i = (int)(t / ((int64_t)n * n));
    const int64_t r = t - (int64_t)i * n * n;
    const int j = (int)(r / n), k = (int)(r - (int64_t)j * n);
    out[t] = mask_bit(m, NB, i, j, k) ? 1 : 0;
  }
}

hipError_t launch_bits_to_bytes(const uint64_t* m, int n, int NB, uint8_t* out, hipStream_t s) {
  const int64_t tot = (int64_t)n * n * n;
  int64_t g = (tot + 255) / 256;
  if (g > 8192) g = 8192;
  hipLaunchKernelGGL(bits_to_bytes_kernel, dim3((unsigned)g), dim3(256), 0, s, m, n, NB, out);
  return hipGetLastError();
}

// ------------------------------------------------------------------ work items from a query list
// For a grid-list decode with per-block token sets: every maximal run of list
// entries in one block is cut into chunks of at most bq queries; n_items counts
// them (the order of items does not affect any result, each query's value depends
// only on its own block's token set). A run of a valid list (unique entries) holds
// at most block^3 entries. An entry outside [0, (R+1)^3) belongs to no block: it
// gets no item, ends the run it interrupts, and its output is set to NaN here.
// One wave per 64 consecutive entries: the lanes compute the entries' blocks at
// once, find the runs that start among them by ballot, and the whole wave looks
// for each run's end 512 entries at a time; the lane of a run's start keeps its
// chunk count, and the item slots of a workgroup's runs are taken with one atomic
// (a serial scan per run by one thread, and an atomic per run, took about 1 ms for
// 720,600 entries in 8^3 blocks; the atomics alone about 0.2 ms in 4^3 blocks).
constexpr int ITEMS_NT = 1024;

__device__ __forceinline__ int list_block(const int32_t* __restrict__ list, int64_t q, int64_t N, int R, int block) {
  if (q < 0 || q >= N) return -2;  // (no entry)
  const unsigned P = (unsigned)R + 1u, lin = (unsigned)list[q];
  if (list[q] < 0 || lin >= P * P * P) return -1;  // (outside the grid; P^3 < 2^31)
  const unsigned i = lin / (P * P), r = lin - i * P * P, j = r / P, k = r - j * P;
  const unsigned NB = ((unsigned)R + (unsigned)block) / (unsigned)block;
  return (int)(((i / block) * NB + j / block) * NB + k / block);
}

__global__ __launch_bounds__(ITEMS_NT) void items_from_list_kernel(const int32_t* __restrict__ list, int64_t N, int R,
                                                                  int block, const int32_t* __restrict__ block_row,
                                                                  int bq, Item* __restrict__ items, int32_t* n_items,
                                                                  float* __restrict__ out) {
  __shared__ int wtot[ITEMS_NT / 64];
  __shared__ int base;
  const int lane = (int)(threadIdx.x & 63), wave = (int)(threadIdx.x >> 6);
  const int64_t seg0 = (int64_t)blockIdx.x * ITEMS_NT + 64 * wave;
  const int64_t q = seg0 + lane;
  int b = -2, nch = 0;  // this lane's block; chunks of the run starting here
  int64_t e = 0;        // ... and that run's end
  if (seg0 < N) {  // (wave-uniform)
    b = list_block(list, q, N, R, block);
    if (b == -1) out[q] = __builtin_nanf("");
    const bool start = b >= 0 && (q == 0 || list_block(list, q - 1, N, R, block) != b);
    for (unsigned long long st = __ballot(start); st; st &= st - 1ull) {
      const int l = __ffsll((long long)st) - 1;
      const int bs = __shfl(b, l);
      // first entry after the start in another block (or past the list)
      unsigned long long d = __ballot(lane > l && b != bs);
      int64_t c = seg0;
      // 8 x 64 entries per step, so that their loads overlap (past N: -2, a mismatch)
      for (int64_t c8 = seg0 + 64; d == 0ull; c8 += 8 * 64) {
        int blks[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) blks[u] = list_block(list, c8 + 64 * u + lane, N, R, block);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const unsigned long long du = __ballot(blks[u] != bs);
          if (d == 0ull && du != 0ull) {
            d = du;
            c = c8 + 64 * u;
          }
        }
      }
      if (lane == l) {
        e = c + __ffsll((long long)d) - 1;
        nch = (int)((e - q + bq - 1) / bq);
      }
    }
  }
  int incl = nch;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o);
    if (lane >= o) incl += u;
  }
  if (lane == 63) wtot[wave] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    int t = 0;
    for (int w = 0; w < ITEMS_NT / 64; ++w) {
      const int v = wtot[w];
      wtot[w] = t;
      t += v;
    }
    base = t > 0 ? atomicAdd(n_items, t) : 0;
  }
  __syncthreads();
  if (nch > 0) {
    const int at = base + wtot[wave] + incl - nch;
    const int row = block_row ? block_row[b] : b;
    (void)VDM_BOUND(row >= 0, BC_LIST_ROW);
    for (int ch = 0; ch < nch; ++ch) {
      const int64_t q0 = q + (int64_t)ch * bq;
      items[at + ch] = Item{(int32_t)q0, (int32_t)min(q0 + bq, e), row, 0};
    }
  }
}

hipError_t launch_items_from_list(const int32_t* list, int64_t N, int R, int block, const int32_t* block_row, int bq,
                                  Item* items, int32_t* n_items, float* out, hipStream_t s) {
  hipLaunchKernelGGL(items_from_list_kernel, dim3((unsigned)((N + ITEMS_NT - 1) / ITEMS_NT)), dim3(ITEMS_NT), 0, s,
                     list, N, R, block, block_row, bq, items, n_items, out);
  return hipGetLastError();
}

VDM_DEBUG_READER(debug_take_hvd)

}  // namespace vdm
