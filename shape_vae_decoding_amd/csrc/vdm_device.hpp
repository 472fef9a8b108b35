// Device-side building blocks shared by the decoder kernels (gfx950 / CDNA4).
//
// MFMA operand layouts used throughout (64-wide wavefront, lane l):
//   A (32 x KS, row-major source X[row][k]):  lane holds X[l % 32][KW*(l / 32) .. +KW-1]
//   B (KS x 32, source Y[col][k] = B^T row-major): lane holds Y[l % 32][KW*(l / 32) .. +KW-1]
//   C (32 x 32, 16 fp32 per lane): register r holds C[crow(r, l)][l % 32],
//       crow(r, l) = 8*(r/4) + 4*(l/32) + r%4
// bf16: v_mfma_f32_32x32x16_bf16 (KW = 8, KS = 16); float: v_mfma_f32_32x32x2_f32
// (KW = 1, KS = 2). Both accumulate in fp32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vdm_internal.hpp"

namespace vdm {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <typename T>
struct Mma;

template <>
struct Mma<bf16> {
  static constexpr int KW = 8;
  static constexpr int KS = 16;
  typedef bf16x8 frag;
  static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <>
struct Mma<float> {
  static constexpr int KW = 1;
  static constexpr int KS = 2;
  typedef float frag;
  static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

// Elements of padding appended to LDS rows (16 bytes) so that 32 lanes reading
// the same column of consecutive rows spread over all banks.
template <typename T>
struct Pad {
  static constexpr int v = 16 / (int)sizeof(T);
};

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// x, hidden from the optimiser: values derived from it are recomputed where they
// are used instead of being hoisted out of a loop and kept live across it.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

__device__ __forceinline__ int crow(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

template <typename T>
__device__ __forceinline__ typename Mma<T>::frag load_frag(const T* base, int ld, int lane) {
  const T* p = base + (lane & 31) * ld + Mma<T>::KW * (lane >> 5);
  return *reinterpret_cast<const typename Mma<T>::frag*>(p);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

template <typename T>
__device__ __forceinline__ T to_t(float x);
template <>
__device__ __forceinline__ bf16 to_t<bf16>(float x) { return (bf16)x; }  // v_cvt_pk_bf16_f32, RNE
template <>
__device__ __forceinline__ float to_t<float>(float x) { return x; }

template <typename T>
__device__ __forceinline__ float to_f(T x) { return (float)x; }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats to a bf16 pair in one v_cvt_pk_bf16_f32 (round to nearest even).
__device__ __forceinline__ bf16x2 cvt2(float a, float b) { return __builtin_convertvector((f32x2){a, b}, bf16x2); }

// Eight floats to the eight bf16 of one MFMA operand fragment.
__device__ __forceinline__ bf16x8 cvt8(const float* x) {
  const bf16x2 a = cvt2(x[0], x[1]), b = cvt2(x[2], x[3]), c = cvt2(x[4], x[5]), d = cvt2(x[6], x[7]);
  const bf16x4 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3);
  const bf16x4 cd = __builtin_shufflevector(c, d, 0, 1, 2, 3);
  return __builtin_shufflevector(ab, cd, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Store 4 consecutive C-layout rows (r = 4g .. 4g+3 of one lane) to dst[0..3].
template <typename T>
__device__ __forceinline__ void store4(T* dst, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4<bf16>(bf16* dst, float a, float b, float c, float d) {
  bf16x4 v;
  v[0] = (bf16)a;
  v[1] = (bf16)b;
  v[2] = (bf16)c;
  v[3] = (bf16)d;
  *reinterpret_cast<bf16x4*>(dst) = v;
}
template <>
__device__ __forceinline__ void store4<float>(float* dst, float a, float b, float c, float d) {
  *reinterpret_cast<f32x4*>(dst) = f32x4{a, b, c, d};
}

// Write one lane's C-tile column as a row: dst[crow(r, l)] = acc[r] (rounded to T).
template <typename T>
__device__ __forceinline__ void store_ct_row(T* dst, const f32x16& acc, int lane) {
  T* p = dst + 4 * (lane >> 5);
#pragma unroll
  for (int g = 0; g < 4; ++g) store4<T>(p + 8 * g, acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]);
}

// Write a 32x32 C tile, transposed, into a row-major [col][row] array:
// dst[(l % 32) * ld + crow(r, l)] = acc[r] (rounded to T).
template <typename T>
__device__ __forceinline__ void store_ct(T* dst, int ld, const f32x16& acc, int lane) {
  store_ct_row<T>(dst + (lane & 31) * ld, acc, lane);
}

// Token order inside a 32-token tile of the packed V^T operand. The P.V product
// takes P from the C layout of S^T = K Q^T: for MFMA step t, lane half h and
// element v it holds C register r = KW*t + v, i.e. key crow(r, h*32). The
// A operand (V^T) must then hold the same keys at the same k slots, so position
// p = KS*t + KW*h + v of a packed V^T row stores token perm_key(p) of the tile.
template <typename T>
__host__ __device__ constexpr int perm_key(int p) {
  constexpr int KW = Mma<T>::KW, KS = Mma<T>::KS;
  const int t = p / KS, h = (p % KS) / KW, v = p % KW, r = KW * t + v;
  return (r & 3) + 8 * (r >> 2) + 4 * h;
}

template <typename T>
__host__ __device__ constexpr int key_pos(int key) {
  for (int p = 0; p < 32; ++p)
    if (perm_key<T>(p) == key) return p;
  return -1;
}

// ------------------------------------------------------------------ geometry

// Grid coordinate of index i on an R-cell grid over [-1,1]: the float32
// quotient of the exact integers (2i - R) and R (correctly rounded division),
// so index 2i of the 2R grid gives the same value as index i of the R grid.
__device__ __forceinline__ float grid_coord(int i, int R) { return (float)(2 * i - R) / (float)R; }

struct Coords {
  float x, y, z;
};

__device__ __forceinline__ Coords grid_point(int64_t lin, int R) {
  const int64_t P = R + 1;
  const int i = (int)(lin / (P * P));
  const int64_t r = lin - (int64_t)i * P * P;
  const int j = (int)(r / P);
  const int k = (int)(r - (int64_t)j * P);
  return Coords{grid_coord(i, R), grid_coord(j, R), grid_coord(k, R)};
}

// Corner probe n (bits: i, j, k choose the high end) of block b: per axis the
// indices block*bx and min(block*bx + block - 1, R).
__device__ __forceinline__ Coords block_corner(int64_t b, int n, int R, int block) {
  const int64_t NB = (R + block) / block;  // ceil((R + 1) / block)
  const int bi = (int)(b / (NB * NB)), bj = (int)((b / NB) % NB), bk = (int)(b % NB);
  auto pick = [&](int bx, int hi) { return hi ? min(block * bx + block - 1, R) : block * bx; };
  return Coords{grid_coord(pick(bi, (n >> 2) & 1), R), grid_coord(pick(bj, (n >> 1) & 1), R),
                grid_coord(pick(bk, n & 1), R)};
}

// The c-th output (from 0) of the SplitMix64 stream seeded with `seed` (Steele,
// Lea and Flood 2014; the mixing constants of Vigna's reference splitmix64.c):
// the state advances by the golden-ratio increment, then is mixed.
__device__ __forceinline__ unsigned long long splitmix64(unsigned long long seed, unsigned long long c) {
  unsigned long long z = seed + (c + 1ull) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Random probe n of block b: along axis a the index lo_a + (u mod e_a), lo_a the
// block's first index, e_a its points along a, u output (8 b + n) * 3 + a of the
// stream.
__device__ __forceinline__ Coords block_random(int64_t b, int n, int R, int block, unsigned long long seed) {
  const int64_t NB = (R + block) / block;
  const int bx[3] = {(int)(b / (NB * NB)), (int)((b / NB) % NB), (int)(b % NB)};
  float c[3];
#pragma unroll
  for (int a = 0; a < 3; ++a) {
    const int lo = block * bx[a];
    const int ext = min(block, R + 1 - lo);
    const unsigned long long u = splitmix64(seed, (unsigned long long)((8 * b + n) * 3 + a));
    c[a] = grid_coord(lo + (int)(u % (unsigned long long)ext), R);
  }
  return Coords{c[0], c[1], c[2]};
}

// Position of query q of a tile's source (points, full grid, grid list, probes).
__device__ __forceinline__ Coords query_coords(const QuerySrc& qs, int64_t q) {
  if (qs.mode == 0) return Coords{qs.xyz[3 * q], qs.xyz[3 * q + 1], qs.xyz[3 * q + 2]};
  if (qs.mode == 3) {
    const int64_t row = q >> 3;
    const int64_t b = qs.list ? (int64_t)qs.list[row] : row;
    return qs.probes ? block_random(b, (int)(q & 7), qs.R, qs.block, qs.seed)
                     : block_corner(b, (int)(q & 7), qs.R, qs.block);
  }
  const int64_t lin = qs.mode == 1 ? q : (int64_t)qs.list[q];
  return grid_point(lin, qs.R);
}

// Analytic SDF of the union of primitives (float32):
// sphere |p - c| - r; box |max(q,0)| + min(max_i q_i, 0) with q = |p - c| - h.
__device__ __forceinline__ float analytic_sdf(Coords p, const PrimSet& ps) {
  float best = __builtin_inff();
  for (int i = 0; i < ps.n; ++i) {
    const PrimDev& pr = ps.p[i];
    const float dx = p.x - pr.c[0], dy = p.y - pr.c[1], dz = p.z - pr.c[2];
    float d;
    if (pr.kind == 0) {
      d = sqrtf(dx * dx + dy * dy + dz * dz) - pr.s[0];
    } else {
      const float qx = fabsf(dx) - pr.s[0], qy = fabsf(dy) - pr.s[1], qz = fabsf(dz) - pr.s[2];
      const float ox = fmaxf(qx, 0.f), oy = fmaxf(qy, 0.f), oz = fmaxf(qz, 0.f);
      d = sqrtf(ox * ox + oy * oy + oz * oz) + fminf(fmaxf(qx, fmaxf(qy, qz)), 0.f);
    }
    best = fminf(best, d);
  }
  return best;
}

// GELU x * Phi(x) = x/2 (1 + erf(x / sqrt 2)), with erf from Abramowitz & Stegun,
// Handbook of Mathematical Functions, formula 7.1.26 (|error| <= 1.5e-7 for all
// arguments; far below the bf16 rounding the hidden activations get next):
// erf(z) = 1 - t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-z^2), t = 1 / (1 + p z), z >= 0.
// With z = |x| / sqrt 2 folded into the constants, and the sign handled by
// x/2 (1 + sign(x) erf|z|) = (x + |x| erf|z|) / 2. Branch-free: one reciprocal
// and one exp2 per value.
__device__ __forceinline__ float gelu(float x) {
  constexpr float P_X = (float)(0.3275911 * 0.70710678118654752);  // p / sqrt 2
  constexpr float C_X = 0.84932180028801904f;                       // sqrt(log2(e) / 2)
  const float ax = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(P_X, ax, 1.f));
  float y = __builtin_fmaf(t, 1.061405429f, -1.453152027f);
  y = __builtin_fmaf(t, y, 1.421413741f);
  y = __builtin_fmaf(t, y, -0.284496736f);
  y = __builtin_fmaf(t, y, 0.254829592f);
  const float u = x * C_X;
  const float e = __builtin_amdgcn_exp2f(-(u * u));  // exp(-x^2 / 2)
  const float erf_abs = __builtin_fmaf(-(t * y), e, 1.f);
  return 0.5f * __builtin_fmaf(ax, erf_abs, x);
}

// ------------------------------------------------------------------ embedding + Q projection

// f_k = 2^k * pi in float32 (float32 pi scaled exactly by 2^k).
__device__ __forceinline__ float freq(int k) { return 3.14159265358979323846f * (float)(1 << k); }

// Fourier features of one axis: e[a] = c, e[3 + 8a + k] = sin(f_k c),
// e[27 + 8a + k] = cos(f_k c), with the float32 product f_k * c as argument.
// `put(index, value)` stores one feature.
template <typename Put>
__device__ __forceinline__ void embed_axis(float c, int a, Put put) {
  put(a, c);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float arg = __fmul_rn(freq(k), c);
    float s, co;
    sincosf(arg, &s, &co);
    put(3 + 8 * a + k, s);
    put(27 + 8 * a + k, co);
  }
}

// MFMA A fragment of Wq [D][51] for rows row0 + (l % 32), features
// ks*KS + KW*(l / 32) + v; features 51..63 read as zero.
template <typename T>
__device__ __forceinline__ typename Mma<T>::frag load_wq_frag(const T* __restrict__ Wq, int row0, int ks, int lane) {
  using MM = Mma<T>;
  const int f0 = ks * MM::KS + MM::KW * (lane >> 5);
  const T* p = Wq + (row0 + (lane & 31)) * VDM_E_DIM;
  // loads stay inside the row (index clamped), then the padding features are zeroed
  if constexpr (MM::KW == 1) {
    const float w = p[f0 < VDM_E_DIM ? f0 : VDM_E_DIM - 1];
    return f0 < VDM_E_DIM ? w : 0.f;
  } else {
    typename MM::frag f;
#pragma unroll
    for (int v = 0; v < MM::KW; ++v) {
      const T w = p[f0 + v < VDM_E_DIM ? f0 + v : VDM_E_DIM - 1];
      f[v] = f0 + v < VDM_E_DIM ? w : to_t<T>(0.f);
    }
    return f;
  }
}

// LDS layout of the embedding / projection stage for a tile of BQ queries.
template <typename T, int BQ, int D>
struct EmbedLds {
  static constexpr int EPAD = 64 + Pad<T>::v;
  static constexpr int DPAD = D + Pad<T>::v;
  static constexpr bool SPLIT = sizeof(T) == 2;  // bf16: features as hi + lo bf16 pairs
  static constexpr int E_HI = 0;
  static constexpr int E_LO = E_HI + BQ * EPAD * (int)sizeof(T);
  static constexpr int QS = E_LO + (SPLIT ? BQ * EPAD * (int)sizeof(T) : 0);
  static constexpr int END = QS + BQ * DPAD * (int)sizeof(T);
};

// Compute Q = Wq e(p) for queries [q0, q1) into Qs[BQ][DPAD] (LDS, rounded to T).
// Rows of queries beyond q1 hold the projection of the origin (never stored).
// bf16: each feature is split into hi + lo bf16 parts and both are projected, so
// the fp32 accumulator carries the product with near-fp32 accuracy before the
// single rounding of Q to bf16.
// Wq: [D][51]. Q is multiplied by qscale before its rounding. Ends with a barrier.
template <typename T, int BQ, int D, int NT>
__device__ __forceinline__ void embed_qproj(const QuerySrc& qs, int64_t q0, int64_t q1, const T* __restrict__ Wq,
                                            char* lds, int tid, float qscale = 1.f) {
  using L = EmbedLds<T, BQ, D>;
  using MM = Mma<T>;
  T* e_hi = reinterpret_cast<T*>(lds + L::E_HI);
  T* e_lo = reinterpret_cast<T*>(lds + L::E_LO);
  T* Qs = reinterpret_cast<T*>(lds + L::QS);
  constexpr int NW = NT / 64;
  static_assert((NW & (NW - 1)) == 0, "a power-of-two number of waves");
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane((tid >> 6) & (NW - 1));
  constexpr int RB = D / 32, CB = BQ / 32, KS = 64 / MM::KS;
  // wave w owns row blocks w, w + NW, .. (RB > NW) or row block w % RB and every
  // (NW / RB)-th column block (RB <= NW); each of its Wq fragments is loaded once
  constexpr int RPW = RB > NW ? RB / NW : 1;
  constexpr int CSTEP = RB > NW ? 1 : NW / RB;
  static_assert(RB % NW == 0 || NW % RB == 0, "row blocks split evenly over waves");
  // the first row block's fragments are issued before the embedding so that
  // their latency overlaps it
  typename MM::frag wq[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) wq[ks] = load_wq_frag<T>(Wq, 32 * (wave % RB), ks, lane);
  for (int idx = tid; idx < BQ * 4; idx += NT) {
    const int qi = idx % BQ;
    const int part = idx / BQ;
    T* hi = e_hi + qi * L::EPAD;
    T* lo = e_lo + qi * L::EPAD;
    auto put = [&](int f, float v) {
      const T h = to_t<T>(v);
      hi[f] = h;
      if constexpr (L::SPLIT) lo[f] = to_t<T>(v - to_f(h));
    };
    if (part == 3) {
      for (int f = 51; f < 64; ++f) put(f, 0.f);
    } else {
      const int64_t q = q0 + qi;
      float c = 0.f;
      if (q < q1) {
        const Coords p = query_coords(qs, q);
        c = part == 0 ? p.x : (part == 1 ? p.y : p.z);
      }
      embed_axis(c, part, put);
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < RPW; ++j) {
    const int rb = RB > NW ? wave + NW * j : wave % RB;
    if (j > 0) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) wq[ks] = load_wq_frag<T>(Wq, 32 * rb, ks, lane);
    }
#pragma unroll
    for (int cb = RB > NW ? 0 : wave / RB; cb < CB; cb += CSTEP) {
      f32x16 acc = zero16();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        acc = MM::mma(wq[ks], load_frag<T>(e_hi + (32 * cb) * L::EPAD + ks * MM::KS, L::EPAD, lane), acc);
        if constexpr (L::SPLIT)
          acc = MM::mma(wq[ks], load_frag<T>(e_lo + (32 * cb) * L::EPAD + ks * MM::KS, L::EPAD, lane), acc);
      }
      acc *= qscale;
      store_ct<T>(Qs + (32 * cb) * L::DPAD + 32 * rb, L::DPAD, acc, lane);
    }
  }
  __syncthreads();
}

}  // namespace vdm
