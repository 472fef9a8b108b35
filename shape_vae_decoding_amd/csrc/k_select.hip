// Adaptive KV Selection on gfx950 (FlashVDM summary, section 4.1 item 2: per
// sub-volume, a few probe queries attend to all latent tokens and the highest
// scoring tokens become the sub-volume's key/value set; techwalker article,
// part 5, describes the same probe-then-reuse scheme).
//
// One workgroup (8 waves) per group of up to 4 blocks: the 32 corner probes of
// the group fill the 32 MFMA columns, so every K tile read serves 4 blocks.
//   pass 1: per (probe, head) softmax max and sum over all tokens (MFMA logits);
//   pass 2: score_j = mean over heads of the softmax probability, written to a
//           per-workgroup scratch row in global memory (32 x M floats do not fit
//           in LDS);
//   top-k:  per probe, the k-th largest score by a bitwise search on the float
//           bits held in registers (scores are >= 0, so unsigned order is float
//           order), then every larger score and the lowest-index equal ones;
//           the block's probes OR their sets into an LDS bitmap;
//   cap:    if the union exceeds `cap`, the cap tokens of largest max-over-probes
//           score (same search; members rank above non-members);
//   output: ascending compaction of the bitmap.
// Each wave covers 1/8 of the tokens in the passes; partial softmax statistics
// are merged in a fixed order, so results are reproducible.
#include <type_traits>

#include "vdm_device.hpp"

namespace vdm {

constexpr int SEL_NT = 512;
constexpr int SEL_NW = SEL_NT / 64;
constexpr int SEL_NP = 8;                // probes per block
constexpr int SEL_GB = 4;                // blocks per workgroup
constexpr int SEL_BQ = SEL_NP * SEL_GB;  // probe columns of the MFMA tile
constexpr int SEL_MAXV = 64;             // scores per lane in the search: M <= 64 * 64
constexpr int SEL_GRID_MAX = 256;        // workgroups (scratch rows are per workgroup)
constexpr int SEL_LIST = 1024;           // per-wave candidate list of the top-k search (LDS)

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o);
    if (lane >= o) v += u;
  }
  return v;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Values u[i] stand for index i * 64 + lane (entries at or past n are 0 and never
// taken). Sets in `bits` the k largest (unsigned order; equal values: lower index
// first). One wave; `list` is its LDS scratch of SEL_LIST values.
//
// The k-th largest value p is the largest threshold with #{u >= p} >= k, built
// bit by bit. For k <= 64 the 64th largest of the lanes' two largest values, lo,
// is a lower bound of p (64 values are >= lo), so only the values >= lo (usually
// a small multiple of k) take part: they are compacted into `list` and the bit
// search runs over 4 (or, for a long list, 16) per lane instead of 48-64; for
// every threshold above lo the counts are the same, and below it both exceed k.
// If more than SEL_LIST values qualify, or k > 64, the search runs over all
// values (3-4 times the work: with the smallest lane maximum as the bound and a
// 256-entry list this path ran for most probes). Thresholds are >= 1, so zero
// entries never count; values are visited in chunks of 16 and a chunk past n is
// skipped.
__device__ __forceinline__ void topk_bits(const unsigned (&u)[SEL_MAXV], int n, int k, unsigned* bits,
                                          unsigned* list, int lane) {
  // (every loop is fully unrolled with constant indices, so u stays in registers)
  constexpr int CH = 16, LV = SEL_LIST / 64;
  static_assert(SEL_MAXV % CH == 0, "whole chunks");
  auto count_all = [&](unsigned thr) {
    int c = 0;
#pragma unroll
    for (int c0 = 0; c0 < SEL_MAXV; c0 += CH) {
      if (c0 * 64 < n) {
#pragma unroll
        for (int i = c0; i < c0 + CH; ++i) c += u[i] >= thr ? 1 : 0;
      }
    }
    return wave_sum(c);
  };
  unsigned p = 0u;
  bool done = false;
  int greater = 0;  // number of values > p (fast path)
  if (k <= 64) {
    // lo = the 64th largest of the 128 values {largest, second largest of each
    // lane}: at least 64 >= k values are >= lo, and it is tighter than the smallest
    // lane maximum (which is <= lo)
    unsigned m1 = 0u, m2 = 0u;
#pragma unroll
    for (int c0 = 0; c0 < SEL_MAXV; c0 += CH) {
      if (c0 * 64 < n) {
#pragma unroll
        for (int i = c0; i < c0 + CH; ++i) {
          const unsigned x = u[i];
          m2 = max(m2, min(m1, x));
          m1 = max(m1, x);
        }
      }
    }
    unsigned lo = 0u;
    for (int b = 31; b >= 0; --b) {
      const unsigned cand = lo | (1u << b);
      if (__popcll(__ballot(m1 >= cand)) + __popcll(__ballot(m2 >= cand)) >= 64) lo = cand;
    }
    int mine = 0;
#pragma unroll
    for (int c0 = 0; c0 < SEL_MAXV; c0 += CH) {
      if (c0 * 64 < n) {
#pragma unroll
        for (int i = c0; i < c0 + CH; ++i) mine += (u[i] >= lo && u[i] > 0u) ? 1 : 0;
      }
    }
    const int incl = wave_incl_scan(mine, lane);
    const int total = __shfl(incl, 63);
    if (lo > 0u && total <= SEL_LIST) {
      int off = incl - mine;
#pragma unroll
      for (int c0 = 0; c0 < SEL_MAXV; c0 += CH) {
        if (c0 * 64 < n) {
#pragma unroll
          for (int i = c0; i < c0 + CH; ++i)
            if (u[i] >= lo) list[off++] = u[i];
        }
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // (counts by ballot and popcount: a short scalar chain per bit instead of a
      // cross-lane reduction; a short list is searched over its first 4 slots per lane)
      auto search = [&](auto lv) {
        constexpr int NV = decltype(lv)::value;
        unsigned v[NV];
#pragma unroll
        for (int j = 0; j < NV; ++j) v[j] = j * 64 + lane < total ? list[j * 64 + lane] : 0u;
        for (int b = 31; b >= 0; --b) {
          const unsigned cand = p | (1u << b);
          int c = 0;
#pragma unroll
          for (int j = 0; j < NV; ++j) c += __popcll(__ballot(v[j] >= cand));
          if (c >= k) p = cand;
        }
        // values > p (all of them are in the list: p >= lo)
        int g = 0;
#pragma unroll
        for (int j = 0; j < NV; ++j) g += __popcll(__ballot(v[j] > p));
        return g;
      };
      greater = total <= 256 ? search(std::integral_constant<int, 4>()) : search(std::integral_constant<int, LV>());
      __builtin_amdgcn_wave_barrier();  // the list is read before the next search writes it
      done = true;
    }
  }
  if (!done) {
    for (int b = 31; b >= 0; --b) {
      const unsigned cand = p | (1u << b);
      if (count_all(cand) >= k) p = cand;
    }
  }
  // copies of p to take, lowest index first
  const int need = k - (done ? greater : (p == 0xffffffffu ? 0 : count_all(p + 1u)));
  int taken = 0;
#pragma unroll
  for (int i = 0; i < SEL_MAXV; ++i) {
    if (i * 64 < n) {
      const int idx = i * 64 + lane;
      const bool valid = idx < n;
      const bool eq = valid && u[i] == p;
      const unsigned long long be = __ballot(eq);
      const int rank = taken + __popcll(be & ((1ull << lane) - 1ull));
      if (valid && (u[i] > p || (eq && rank < need))) atomicOr(&bits[idx >> 5], 1u << (idx & 31));
      taken += __popcll(be);
    }
  }
}

// LDS: [embedding stage] | stats [NW][H][32] float2 | lists [NW][SEL_LIST] | bits [GB][words] |
//      bits2 [GB][words] | cnt [GB]
template <typename T, int H>
struct SelCfg {
  static constexpr int D = 64 * H;
  static constexpr int EMB_END = EmbedLds<T, SEL_BQ, D>::END;
  static constexpr int STATS = (EMB_END + 15) & ~15;
  static constexpr int LISTS = STATS + SEL_NW * H * 32 * 8;
  static constexpr int BITS = LISTS + SEL_NW * SEL_LIST * 4;
  __host__ __device__ static int total(int M) {
    const int words = (M + 31) / 32;
    return BITS + 2 * SEL_GB * words * 4 + SEL_GB * 4 + 16;
  }
};

// per-workgroup scratch: SEL_BQ rows of Mpad scores
__host__ __device__ inline int sel_mpad(int M) { return (M + 63) / 64 * 64; }

// Scores row r, element i * 64 + lane, for i = 0 .. SEL_MAXV-1, as unsigned bits
// (0 past M). Buffer loads: a scalar offset per i, so no per-element address
// registers are kept live.
__device__ __forceinline__ void load_scores(__amdgpu_buffer_rsrc_t buf, int row, int Mp, int M, int lane,
                                            unsigned (&u)[SEL_MAXV]) {
  const int voff = (row * Mp + lane) * 4;
#pragma unroll
  for (int i = 0; i < SEL_MAXV; ++i) {
    const unsigned v = __builtin_amdgcn_raw_buffer_load_b32(buf, voff, i * 256, 0);
    u[i] = i * 64 + lane < M ? v : 0u;
  }
}

// K fragments of key tile kb for every head (A operands of S^T = K Q^T). bf16:
// from the packed tiles, each load one contiguous 1 KB (chunk ks of head h);
// fp32: from the rows of K (keys past M clamped; their logits are masked).
template <typename T, int H>
struct KTile {
  using Frag = typename Mma<T>::frag;
  static constexpr int KS_H = 64 / Mma<T>::KS;
  Frag f[H][KS_H];
};

template <typename T, int H>
__device__ __forceinline__ void load_ktile(const SelectArgs& A, __amdgpu_buffer_rsrc_t kbuf, int kb, int lane,
                                           KTile<T, H>& t) {
  using MM = Mma<T>;
  using Frag = typename MM::frag;
  constexpr int KS_H = KTile<T, H>::KS_H;
  if constexpr (sizeof(T) == 2) {
    static_assert(KS_H * 16 == 32 * (int)sizeof(T), "one 16-byte chunk of the packed run per MFMA step");
#pragma unroll
    for (int h = 0; h < H; ++h)
#pragma unroll
      for (int ks = 0; ks < KS_H; ++ks) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(kbuf, lane * 16, ((kb * H + h) * KS_H + ks) * 1024, 0);
        const uint4 u{v[0], v[1], v[2], v[3]};
        t.f[h][ks] = *reinterpret_cast<const Frag*>(&u);
      }
  } else {
    const int key = min(kb * 32 + (lane & 31), A.M - 1);
    const T* krow = (const T*)A.K + (int64_t)key * (64 * H) + MM::KW * (lane >> 5);
#pragma unroll
    for (int h = 0; h < H; ++h)
#pragma unroll
      for (int ks = 0; ks < KS_H; ++ks) t.f[h][ks] = *reinterpret_cast<const Frag*>(krow + 64 * h + ks * MM::KS);
  }
}

template <typename T, int H>
__global__ __launch_bounds__(SEL_NT) void select_kernel(SelectArgs A) {
  extern __shared__ __align__(16) char lds[];
  using MM = Mma<T>;
  using Frag = typename MM::frag;
  using L = EmbedLds<T, SEL_BQ, 64 * H>;
  using CF = SelCfg<T, H>;
  constexpr int D = 64 * H, KS_H = 64 / MM::KS;
  const int tid0 = threadIdx.x, lane0 = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid0 >> 6);
  const int M = A.M, Mp = sel_mpad(M);
  const int nwords = (M + 31) / 32;
  float2* stats = reinterpret_cast<float2*>(lds + CF::STATS);     // [NW][H][32]
  unsigned* bits = reinterpret_cast<unsigned*>(lds + CF::BITS);    // [GB][nwords]
  unsigned* bits2 = bits + SEL_GB * nwords;                        // [GB][nwords]
  int* ucount = reinterpret_cast<int*>(bits2 + SEL_GB * nwords);   // [GB]
  float* scores = A.scores + (int64_t)blockIdx.x * SEL_BQ * Mp;    // [BQ][Mp], this workgroup's rows
  unsigned* wlist = reinterpret_cast<unsigned*>(lds + CF::LISTS) + wave * SEL_LIST;  // this wave's top-k list
  const __amdgpu_buffer_rsrc_t sbuf =
      __builtin_amdgcn_make_buffer_rsrc(scores, (short)0, SEL_BQ * Mp * 4, 0x00020000 /* raw buffer */);
  const int64_t nblk = A.d_n_blocks ? (int64_t)*A.d_n_blocks : A.n_blocks;
  const int64_t ngroups = (nblk + SEL_GB - 1) / SEL_GB;
  const __amdgpu_buffer_rsrc_t kbuf =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(A.Kp), (short)0, sizeof(T) == 2 ? (M + 31) / 32 * 32 * D * 2 : 0,
                                        0x00020000 /* raw buffer */);
  QuerySrc qs;
  qs.mode = 3;
  qs.R = A.R;
  qs.xyz = nullptr;
  qs.list = A.blocks;
  qs.block = A.block;
  qs.probes = A.probes;
  qs.seed = A.seed;
  const int nkb = (M + 31) / 32;
  const int per = (nkb + SEL_NW - 1) / SEL_NW;
  const int kb0 = wave * per, kb1 = min(nkb, kb0 + per);
  const float NEG = -__builtin_inff();

  for (int64_t grp = blockIdx.x; grp < ngroups; grp += gridDim.x) {
    const int64_t row0 = grp * SEL_GB;
    const int nb = (int)min<int64_t>(SEL_GB, nblk - row0);
    // thread and lane indices re-derived opaquely per phase, so the address
    // arithmetic of a phase is not hoisted out of the group loop (and kept live
    // across the other phases)
    int tid = opaque(tid0), lane = opaque(lane0);
    int col = lane & 31;  // this lane's probe (MFMA column)
    embed_qproj<T, SEL_BQ, D, SEL_NT>(qs, row0 * SEL_NP, (row0 + nb) * SEL_NP, (const T*)A.Wq, lds, tid);
    const T* qrow = reinterpret_cast<const T*>(lds + L::QS) + col * L::DPAD + MM::KW * (lane >> 5);
    // this wave's key tiles kb0 .. kb1-1, two at a time with static fragment buffers
    auto over_key_tiles = [&](auto&& work) {
      if (kb0 >= kb1) return;
      KTile<T, H> ta, tb;
      load_ktile<T, H>(A, kbuf, kb0, lane, ta);
      int kb = kb0;
      for (; kb + 1 < kb1; kb += 2) {
        load_ktile<T, H>(A, kbuf, kb + 1, lane, tb);
        work(ta, kb);
        load_ktile<T, H>(A, kbuf, kb + 2 < kb1 ? kb + 2 : kb1 - 1, lane, ta);
        work(tb, kb + 1);
      }
      if (kb < kb1) work(ta, kb);
    };

    // ---------------------------------------------------------------- pass 1: softmax statistics
    float m[H], l[H];
#pragma unroll
    for (int h = 0; h < H; ++h) {
      m[h] = NEG;
      l[h] = 0.f;
    }
    // (key tiles in pairs, the next tile's fragments loaded beside the current one's work)
    auto stats_tile = [&](const KTile<T, H>& t, int kb) {
#pragma unroll
      for (int h = 0; h < H; ++h) {
        f32x16 S = zero16();
#pragma unroll
        for (int ks = 0; ks < KS_H; ++ks)
          S = MM::mma(t.f[h][ks], *reinterpret_cast<const Frag*>(qrow + 64 * h + ks * MM::KS), S);
        float mx = NEG;
        float tt[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) tt[r] = S[r] * 0.18033688011112042f;
        if (kb * 32 + 32 > M) {  // (uniform) the last, partial tile: keys past M do not count
#pragma unroll
          for (int r = 0; r < 16; ++r) tt[r] = kb * 32 + crow(r, lane) < M ? tt[r] : NEG;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, tt[r]);
        const float mnew = fmaxf(m[h], mx);
        if (mnew != NEG) {
          float sum = 0.f;
#pragma unroll
          for (int r = 0; r < 16; ++r) sum += __builtin_amdgcn_exp2f(tt[r] - mnew);
          l[h] = l[h] * __builtin_amdgcn_exp2f(m[h] - mnew) + sum;
          m[h] = mnew;
        }
      }
    };
    over_key_tiles(stats_tile);
#pragma unroll
    for (int h = 0; h < H; ++h) {
      const float mo = __shfl_xor(m[h], 32), lo = __shfl_xor(l[h], 32);
      const float mm = fmaxf(m[h], mo);
      if (mm != NEG) {
        l[h] = l[h] * __builtin_amdgcn_exp2f(m[h] - mm) + lo * __builtin_amdgcn_exp2f(mo - mm);
        m[h] = mm;
      }
      if (lane < 32) stats[(wave * H + h) * 32 + lane] = make_float2(m[h], l[h]);
    }
    for (int i = tid; i < 2 * SEL_GB * nwords; i += SEL_NT) bits[i] = 0u;
    __syncthreads();
    float mf[H], linv[H];
#pragma unroll
    for (int h = 0; h < H; ++h) {
      float mm = NEG, ll = 0.f;
      for (int w = 0; w < SEL_NW; ++w) {
        const float2 st = stats[(w * H + h) * 32 + col];
        const float mn = fmaxf(mm, st.x);
        if (mn != NEG) {
          ll = ll * __builtin_amdgcn_exp2f(mm - mn) + st.y * __builtin_amdgcn_exp2f(st.x - mn);
          mm = mn;
        }
      }
      mf[h] = mm;
      linv[h] = 1.f / ll;
    }

    // ---------------------------------------------------------------- pass 2: head-mean probabilities
    lane = opaque(lane);
    col = lane & 31;
    auto score_tile = [&](const KTile<T, H>& t, int kb) {
      float acc[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
      for (int h = 0; h < H; ++h) {
        f32x16 S = zero16();
#pragma unroll
        for (int ks = 0; ks < KS_H; ++ks)
          S = MM::mma(t.f[h][ks], *reinterpret_cast<const Frag*>(qrow + 64 * h + ks * MM::KS), S);
#pragma unroll
        for (int r = 0; r < 16; ++r)
          acc[r] += __builtin_amdgcn_exp2f(S[r] * 0.18033688011112042f - mf[h]) * linv[h];
      }
      if (col < nb * SEL_NP) {
        const bool full = kb * 32 + 32 <= M;  // (uniform)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = kb * 32 + crow(r, lane);
          if (full || j < M) scores[col * Mp + j] = acc[r] * (1.f / H);
        }
      }
    };
    over_key_tiles(score_tile);
    __syncthreads();  // the scores rows are complete and visible to the workgroup

    // ---------------------------------------------------------------- top-k per probe, union per block
    tid = opaque(tid);
    lane = opaque(lane);
    for (int p = wave; p < nb * SEL_NP; p += SEL_NW) {
      unsigned u[SEL_MAXV];
      load_scores(sbuf, p, Mp, M, lane, u);
      topk_bits(u, M, A.k, bits + (p / SEL_NP) * nwords, wlist, lane);
    }
    __syncthreads();

    // ---------------------------------------------------------------- cap, compaction (one wave per block)
    tid = opaque(tid);
    lane = opaque(lane);
    if (wave < nb) {
      const int blk = wave;
      unsigned* ub = bits + blk * nwords;
      int cnt = 0;
      for (int i = lane; i < nwords; i += 64) cnt += __popc(ub[i]);
      cnt = wave_sum(cnt);
      const unsigned* outbits = ub;
      if (cnt > A.cap) {
        // keep the cap tokens of largest max-over-probes score (members rank above non-members)
        unsigned u[SEL_MAXV];
        load_scores(sbuf, blk * SEL_NP, Mp, M, lane, u);
        for (int q = 1; q < SEL_NP; ++q) {
          const int voff = ((blk * SEL_NP + q) * Mp + lane) * 4;
#pragma unroll
          for (int i = 0; i < SEL_MAXV; ++i)  // scores >= 0: bit order is float order
            u[i] = max(u[i], __builtin_amdgcn_raw_buffer_load_b32(sbuf, voff, i * 256, 0));
        }
#pragma unroll
        for (int i = 0; i < SEL_MAXV; ++i) {
          const int idx = i * 64 + lane;
          const bool member = idx < M && ((ub[idx >> 5] >> (idx & 31)) & 1u);
          u[i] = member ? u[i] + 1u : 0u;
        }
        topk_bits(u, M, A.cap, bits2 + blk * nwords, wlist, lane);
        outbits = bits2 + blk * nwords;
      }
      const int64_t row = row0 + blk;
      int32_t* out = A.sel_idx + row * (int64_t)A.cap;
      int base = 0;
      for (int w0 = 0; w0 < nwords; w0 += 64) {
        const int wi = w0 + lane;
        unsigned word = wi < nwords ? outbits[wi] : 0u;
        const int c = __popc(word);
        const int incl = wave_incl_scan(c, lane);
        int off = base + incl - c;
        while (word) {
          const int b = __ffs(word) - 1;
          out[off++] = wi * 32 + b;
          word &= word - 1u;
        }
        base += __shfl(incl, 63);
      }
      for (int i = base + lane; i < A.cap; i += 64) out[i] = -1;
      if (lane == 0) {
        A.sel_cnt[row] = base;
        ucount[blk] = base;
      }
    }
    __syncthreads();
    if (tid == 0 && A.stat_selected) {
      int64_t t = 0;
      for (int b = 0; b < nb; ++b) t += ucount[b];
      atomicAdd((unsigned long long*)A.stat_selected, (unsigned long long)t);
    }
  }
}

template <typename T, int H>
static hipError_t run_select(const SelectArgs& a, hipStream_t s) {
  const int lds = SelCfg<T, H>::total(a.M);
  const void* fn = reinterpret_cast<const void*>(&select_kernel<T, H>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  int64_t grid = dev_info().cus;
  if (grid > SEL_GRID_MAX) grid = SEL_GRID_MAX;
  if (!a.d_n_blocks) {
    const int64_t groups = (a.n_blocks + SEL_GB - 1) / SEL_GB;
    if (groups < grid) grid = groups;
  }
  if (grid < 1) return hipSuccess;
  hipLaunchKernelGGL((select_kernel<T, H>), dim3((unsigned)grid), dim3(SEL_NT), lds, s, a);
  return hipGetLastError();
}

size_t select_scratch_bytes(int M) { return (size_t)SEL_GRID_MAX * SEL_BQ * sel_mpad(M) * sizeof(float); }

hipError_t launch_select(int dtype, const SelectArgs& a, hipStream_t s) {
  if (a.M > SEL_MAXV * 64) return hipErrorInvalidValue;
  if (dtype == VDM_BF16) return a.D == 256 ? run_select<bf16, 4>(a, s) : run_select<bf16, 1>(a, s);
  return run_select<float, 1>(a, s);
}

}  // namespace vdm
