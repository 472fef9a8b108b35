// Adaptive KV Selection on gfx950 (FlashVDM summary, section 4.1 item 2: per
// sub-volume, a few probe queries attend to all latent tokens and the highest
// scoring tokens become the sub-volume's key/value set; techwalker article,
// part 5, describes the same probe-then-reuse scheme).
//
// One workgroup (8 waves) per group of up to 4 blocks: the 32 corner probes of
// the group fill the 32 MFMA columns, so every K tile read serves 4 blocks.
//   pass 1: per (probe, head) softmax max and sum over all tokens (MFMA logits
//           as K Q^T: one probe per lane, so the statistics are per-lane sums);
//   pass 2: score_j = mean over heads of the softmax probability, 1/sum folded
//           into the exponent; the logits are formed as Q K^T (16 probes and one
//           token per lane), so each store writes 32 consecutive tokens of a
//           probe's row in the per-workgroup scratch (32 x M floats do not fit in
//           LDS);
//   top-k:  per probe, the k-th largest score by a bitwise search on the float
//           bits held in registers (scores are >= 0, so unsigned order is float
//           order), then every larger score and the lowest-index equal ones, as a
//           per-lane mask; a wave ORs the masks of its probes of one block and
//           adds them to the block's LDS bitmap with one ballot per mask bit;
//   cap:    if the union exceeds `cap`, the cap tokens of largest max-over-probes
//           score (same search; members rank above non-members);
//   output: ascending compaction of the bitmap.
// Per-head sets (PH): pass 2 keeps each head's probability as its own score row,
// and top-k, union, cap and output run per (block, head).
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
constexpr int SEL_LSTRIDE = SEL_LIST + 64;  // ... and one discard slot per lane after it
constexpr int SEL_MAX_M = 65536;         // tokens of a selection (one set per block)
constexpr int SEL_MAX_M_PH = 16384;      // tokens of a per-head selection (4 score rows per probe)
constexpr int SEL_CHUNK = SEL_MAXV * 64; // tokens per search of a chunked row
constexpr int SEL_CV = SEL_LIST / 64;    // list entries per lane

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
// taken). Returns the lane's mask of the k largest (bit i: value i of this lane;
// unsigned order; equal values: lower index first). One wave; `list` is its LDS
// scratch of SEL_LSTRIDE values (SEL_LIST, then a discard slot per lane).
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
// skipped. Within a chunk nothing branches (a branch per value ends the
// scheduling region): entries past n are 0, so they fail every comparison with
// a positive threshold, and the list is filled by writing every value, those
// below lo to the lane's discard slot.
template <int NU>
__device__ __forceinline__ uint64_t topk_mask(const unsigned (&u)[NU], int n, int k, unsigned* list, int lane) {
  // (every loop is fully unrolled with constant indices, so u stays in registers)
  constexpr int CH = 16, LV = SEL_LIST / 64;
  static_assert(NU % CH == 0, "whole chunks");
  auto count_all = [&](unsigned thr) {
    int c = 0;
#pragma unroll
    for (int c0 = 0; c0 < NU; c0 += CH) {
      if (c0 * 64 < n) {
#pragma unroll
        for (int i = c0; i < c0 + CH; ++i) c += u[i] >= thr ? 1 : 0;
      }
    }
    return wave_sum(c);
  };
  unsigned p = 0u;
  bool done = false;
  int greater = 0, equal = 0;  // numbers of values > p and == p (fast path)
  if (k <= 64) {
    // lo = the 64th largest of the 128 values {largest, second largest of each
    // lane}: at least 64 >= k values are >= lo, and it is tighter than the smallest
    // lane maximum (which is <= lo)
    unsigned m1 = 0u, m2 = 0u;
#pragma unroll
    for (int c0 = 0; c0 < NU; c0 += CH) {
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
    const unsigned lo1 = max(lo, 1u);
    int mine = 0;
#pragma unroll
    for (int c0 = 0; c0 < NU; c0 += CH) {
      if (c0 * 64 < n) {
#pragma unroll
        for (int i = c0; i < c0 + CH; ++i) mine += u[i] >= lo1 ? 1 : 0;
      }
    }
    const int incl = wave_incl_scan(mine, lane);
    const int total = __shfl(incl, 63);
    if (lo > 0u && total <= SEL_LIST) {
      int off = incl - mine;
      const int discard = SEL_LIST + lane;
#pragma unroll
      for (int c0 = 0; c0 < NU; c0 += CH) {
        if (c0 * 64 < n) {
#pragma unroll
          for (int i = c0; i < c0 + CH; ++i) {
            const bool in = u[i] >= lo;
            list[in ? off : discard] = u[i];
            off += in ? 1 : 0;
          }
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
        // values > p and == p (all of them are in the list: p >= lo)
        int g = 0, e = 0;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
          g += __popcll(__ballot(v[j] > p));
          e += __popcll(__ballot(v[j] == p));
        }
        return make_int2(g, e);
      };
      const int2 ge = total <= 256 ? search(std::integral_constant<int, 4>()) : search(std::integral_constant<int, LV>());
      greater = ge.x;
      equal = ge.y;
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
  if (!done) {
    greater = p == 0xffffffffu ? 0 : count_all(p + 1u);
    equal = count_all(p) - greater;
  }
  // copies of p to take, lowest index first; usually every copy (no tie at the cut)
  const int need = k - greater;
  // (the mask in two 32-bit halves: constant shifts, no 64-bit shifts per value)
  unsigned sel[2] = {0u, 0u};
  if (p > 0u && equal == need) {
#pragma unroll
    for (int c0 = 0; c0 < NU; c0 += CH) {
      if (c0 * 64 < n) {
#pragma unroll
        for (int i = c0; i < c0 + CH; ++i) sel[i >> 5] |= u[i] >= p ? 1u << (i & 31) : 0u;  // (past n: 0 < p)
      }
    }
    return (uint64_t)sel[1] << 32 | sel[0];
  }
  // (ties at the cut, rare: entries past n are 0, so only a cut of 0 needs the
  // index test; the lane comes through an opaque copy so that those 64 compares
  // are not hoisted out of the callers' loops, where they took 64 VGPRs and 128
  // spilled SGPRs)
  int taken = 0;
  const int ln = opaque(lane);
  const uint64_t below = (1ull << ln) - 1ull;
  const bool zero_cut = p == 0u;
#pragma unroll
  for (int c0 = 0; c0 < NU; c0 += CH) {
    if (c0 * 64 < n) {
#pragma unroll
      for (int i = c0; i < c0 + CH; ++i) {
        const bool valid = !zero_cut || i * 64 + ln < n;
        const bool eq = valid && u[i] == p;
        const unsigned long long be = __ballot(eq);
        const int rank = taken + __popcll(be & below);
        sel[i >> 5] |= valid && (u[i] > p || (eq && rank < need)) ? 1u << (i & 31) : 0u;
        taken += __popcll(be);
      }
    }
  }
  return (uint64_t)sel[1] << 32 | sel[0];
}

// Adds a wave's selection masks (bit i of lane l: token i * 64 + l) to a bitmap of
// 32-bit words (token t: bit t % 32 of word t / 32; 8-byte aligned): the ballot of
// bit i is words 2i and 2i+1. Lane i collects that ballot, then every
// lane with a nonzero word ORs it in: one LDS atomic per lane, no branch per bit.
__device__ __forceinline__ void add_to_bitmap(uint64_t sel, int n, unsigned* words, int lane) {
  const unsigned s0 = (unsigned)sel, s1 = (unsigned)(sel >> 32);
  int w0 = 0, w1 = 0;
  lane = opaque(lane);  // (the 64 tests lane == i are not hoisted into spilled scalar masks)
#pragma unroll
  for (int c0 = 0; c0 < SEL_MAXV; c0 += 16) {
    if (c0 * 64 < n) {
#pragma unroll
      for (int i = c0; i < c0 + 16; ++i) {
        const unsigned long long b = __ballot(((i < 32 ? s0 : s1) >> (i & 31)) & 1u);
        w0 = lane == i ? (int)(unsigned)b : w0;
        w1 = lane == i ? (int)(unsigned)(b >> 32) : w1;
      }
    }
  }
  const unsigned long long w = (unsigned long long)(unsigned)w1 << 32 | (unsigned)w0;
  if (w != 0ull) atomicOr(reinterpret_cast<unsigned long long*>(words) + lane, w);
}

// LDS: [embedding stage] | stats [NW][H][32] float2 | fin [H][32] | lists [NW][SEL_LSTRIDE] |
//      bits [GB*NS][wst] | bits2 [GB*NS][wst] | cnt [GB*NS] | (cand [NW][SEL_LIST])
//      (NS sets per block: H with per-head sets, else 1; wst = sel_wstride(M) words
//      per set, an even number). Chunked rows (M > SEL_CHUNK) keep each wave's token
//      list in `cand`: over the embedding stage and stats, which are dead once pass 2
//      has ended, where they are large enough, else past the counts.
__host__ __device__ constexpr int sel_wstride(int M) { return 2 * ((M + 63) / 64); }

template <typename T, int H, int NS>
struct SelCfg {
  static constexpr int D = 64 * H;
  static constexpr int EMB_END = EmbedLds<T, SEL_BQ, D>::END;
  static constexpr int STATS = (EMB_END + 15) & ~15;
  static constexpr int FIN = STATS + SEL_NW * H * 32 * 8;
  static constexpr int LISTS = FIN + H * 32 * 4;
  static constexpr int BITS = LISTS + SEL_NW * SEL_LSTRIDE * 4;
  static constexpr int CAND_BYTES = SEL_NW * SEL_LIST * 4;
  static constexpr bool CAND_LOW = FIN >= CAND_BYTES;
  static_assert(BITS % 16 == 0, "16-byte aligned bitmaps");
  static_assert(SEL_LIST >= 32 * 32, "a wave's list holds its 32 x 32 transposition tile in pass 2");
  __host__ __device__ static constexpr int bits_end(int M) {
    return BITS + 2 * SEL_GB * NS * sel_wstride(M) * 4 + SEL_GB * NS * 4 + 16;
  }
  __host__ __device__ static constexpr int cand(int M) { return CAND_LOW ? 0 : (bits_end(M) + 15) & ~15; }
  __host__ __device__ static constexpr int total(int M) {
    return M > SEL_CHUNK && !CAND_LOW ? cand(M) + CAND_BYTES : bits_end(M);
  }
};

constexpr int SEL_LDS_MAX = 160 * 1024;
static_assert(SelCfg<bf16, 4, 1>::total(SEL_MAX_M) <= SEL_LDS_MAX && SelCfg<bf16, 4, 4>::total(SEL_MAX_M_PH) <= SEL_LDS_MAX &&
                  SelCfg<bf16, 1, 1>::total(SEL_MAX_M) <= SEL_LDS_MAX && SelCfg<float, 1, 1>::total(SEL_MAX_M) <= SEL_LDS_MAX,
              "the largest selections fit the LDS of a workgroup");

// per-workgroup scratch: SEL_BQ rows of Mpad scores
__host__ __device__ inline int sel_mpad(int M) { return (M + 63) / 64 * 64; }

// Scores row r (of the rows starting at `scores`, Mp apart), element c0 + i * 64 +
// lane, for i = 0 .. SEL_MAXV-1, as unsigned bits. The buffer covers the row's M
// values only, so loads past M return 0 without touching memory. Buffer loads: a
// scalar offset per i, so no per-element address registers are kept live.
__device__ __forceinline__ void load_scores(const float* scores, int row, int Mp, int M, int lane,
                                            unsigned (&u)[SEL_MAXV], int c0 = 0) {
  const __amdgpu_buffer_rsrc_t buf = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(scores) + (int64_t)row * Mp, (short)0, M * 4, 0x00020000 /* raw buffer */);
  const int voff = (c0 + lane) * 4;
#pragma unroll
  for (int i = 0; i < SEL_MAXV; ++i) u[i] = __builtin_amdgcn_raw_buffer_load_b32(buf, voff, i * 256, 0);
}

// Rows of more than SEL_MAXV * 64 tokens are searched in chunks of that many. A
// token among the k largest of the row (equal scores: lower index first) is among
// the k largest of its chunk by the same order, so the chunks' winners, kept in
// ascending token order, hold the row's k largest with the same tie order; a
// second search over them (at most SEL_LIST, so NV = 16 per lane) picks those.

// Appends the tokens of a chunk's mask (bit i of lane l: token c0 + i * 64 + l) to
// a wave's list in ascending order; returns the new length.
__device__ __forceinline__ int append_tokens(uint64_t sel, int c0, int n, int* list, int len, int lane) {
  const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
  for (int i = 0; i < SEL_MAXV; ++i) {
    if (i * 64 < n) {
      const bool on = (sel >> i) & 1ull;
      const unsigned long long b = __ballot(on);
      const int slot = len + __popcll(b & below);
      if (on && VDM_BOUND(slot < SEL_LIST, BC_SELECT_CAND)) list[slot] = c0 + i * 64 + lane;
      len += __popcll(b);
    }
  }
  return len;
}

// Sets the bits of the tokens list[j * 64 + lane] whose bit j of `sel` is set.
__device__ __forceinline__ void mark_listed(uint64_t sel, const int* list, unsigned* words, int lane) {
#pragma unroll
  for (int j = 0; j < SEL_CV; ++j)
    if ((sel >> j) & 1ull) {
      const int t = list[j * 64 + lane];
      atomicOr(words + (t >> 5), 1u << (t & 31));
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
__device__ __forceinline__ void load_ktile(const SelectArgs& A, const void* Kraw, __amdgpu_buffer_rsrc_t kbuf, int kb,
                                           int lane, KTile<T, H>& t) {
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
    const T* krow = (const T*)Kraw + (int64_t)key * (64 * H) + MM::KW * (lane >> 5);
#pragma unroll
    for (int h = 0; h < H; ++h)
#pragma unroll
      for (int ks = 0; ks < KS_H; ++ks) t.f[h][ks] = *reinterpret_cast<const Frag*>(krow + 64 * h + ks * MM::KS);
  }
}

// RG: a ragged batch of shapes (grp_prefix); a separate instance, so that the
// single-shape kernels keep their registers.
template <typename T, int H, bool PH, bool BIG, bool RG>
__global__ __launch_bounds__(SEL_NT) void select_kernel(SelectArgs A) {
  extern __shared__ __align__(16) char lds[];
  using MM = Mma<T>;
  using Frag = typename MM::frag;
  using L = EmbedLds<T, SEL_BQ, 64 * H>;
  constexpr int NS = PH ? H : 1;  // token sets (and score rows per probe) per block
  using CF = SelCfg<T, H, NS>;
  constexpr int D = 64 * H, KS_H = 64 / MM::KS;
  const int tid0 = threadIdx.x, lane0 = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid0 >> 6);
  const int M = A.M, Mp = sel_mpad(M);
  const int nwords = (M + 31) / 32, wst = sel_wstride(M);
  float2* stats = reinterpret_cast<float2*>(lds + CF::STATS);       // [NW][H][32]
  float* fin = reinterpret_cast<float*>(lds + CF::FIN);             // [H][32]
  unsigned* bits = reinterpret_cast<unsigned*>(lds + CF::BITS);     // [GB][NS][wst]
  unsigned* bits2 = bits + SEL_GB * NS * wst;                       // [GB][NS][wst]
  int* ucount = reinterpret_cast<int*>(bits2 + SEL_GB * NS * wst);  // [GB][NS]
  float* scores = A.scores + (int64_t)blockIdx.x * SEL_BQ * NS * Mp;   // [BQ][NS][Mp], this workgroup's rows
  unsigned* wlist = reinterpret_cast<unsigned*>(lds + CF::LISTS) + wave * SEL_LSTRIDE;  // this wave's top-k list
  int* cand = reinterpret_cast<int*>(lds + CF::cand(M)) + wave * SEL_LIST;          // chunked rows: token list
  const __amdgpu_buffer_rsrc_t sbuf =
      __builtin_amdgcn_make_buffer_rsrc(scores, (short)0, SEL_BQ * NS * Mp * 4, 0x00020000 /* raw buffer */);
  const int64_t nblk_all = A.d_n_blocks ? (int64_t)*A.d_n_blocks : A.n_blocks;
  const int64_t ngroups = RG ? A.grp_prefix[A.batch] : (nblk_all + SEL_GB - 1) / SEL_GB;
  // a shape's inputs (RG: per group; otherwise shape 0's, once)
  struct In {
    const int32_t* blocks;
    const void* Kraw;
    int32_t* sel_idx;
    int32_t* sel_cnt;
    int64_t* stat_selected;
    __amdgpu_buffer_rsrc_t kbuf;
  };
  auto inputs_of = [&](int shape) {
    auto at = [&](auto* p, int64_t stride) { return (decltype(p))((char*)p + shape * stride); };
    In in;
    in.blocks = A.blocks ? at(A.blocks, A.blocks_stride) : nullptr;
    in.Kraw = at(A.K, A.k_stride);
    in.sel_idx = at(A.sel_idx, A.sel_stride);
    in.sel_cnt = at(A.sel_cnt, A.sel_stride);
    in.stat_selected = A.stat_selected ? at(A.stat_selected, A.stat_stride) : nullptr;
    in.kbuf = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(at(A.Kp, A.kp_stride)), (short)0,
                                                sizeof(T) == 2 ? (M + 31) / 32 * 32 * D * 2 : 0,
                                                0x00020000 /* raw buffer */);
    return in;
  };
  const In in0 = inputs_of(0);
  const int nkb = (M + 31) / 32;
  const int per = (nkb + SEL_NW - 1) / SEL_NW;
  const int kb0 = wave * per, kb1 = min(nkb, kb0 + per);
  const float NEG = -__builtin_inff();

  for (int64_t grp = blockIdx.x; grp < ngroups; grp += gridDim.x) {
    // this group's shape (ragged batch: grp_prefix[shape] <= grp < grp_prefix[shape + 1];
    // a shape without blocks has equal neighbours and is passed over) and its inputs
    int64_t lgrp = grp, nblk = nblk_all;
    In in = in0;
    if constexpr (RG) {
      int lo = 0;
#pragma unroll
      for (int step = 2048; step >= 1; step >>= 1) {  // (batches of at most 4096 shapes)
        const int mid = lo + step;
        lo = mid < A.batch && A.grp_prefix[mid] <= grp ? mid : lo;
      }
      const int shape = __builtin_amdgcn_readfirstlane(lo);
      lgrp = grp - A.grp_prefix[shape];
      nblk = A.d_n_blocks[shape * A.cnt_stride];
      in = inputs_of(shape);
    }
    const int32_t* blocks = in.blocks;
    const void* Kraw = in.Kraw;
    int32_t* sel_idx = in.sel_idx;
    int32_t* sel_cnt = in.sel_cnt;
    int64_t* stat_selected = in.stat_selected;
    const __amdgpu_buffer_rsrc_t kbuf = in.kbuf;
    QuerySrc qs;
    qs.mode = 3;
    qs.R = A.R;
    qs.xyz = nullptr;
    qs.list = blocks;
    qs.block = A.block;
    qs.probes = A.probes;
    qs.seed = A.seed;
    const int64_t row0 = lgrp * SEL_GB;
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
      load_ktile<T, H>(A, Kraw, kbuf, kb0, lane, ta);
      int kb = kb0;
      for (; kb + 1 < kb1; kb += 2) {
        load_ktile<T, H>(A, Kraw, kbuf, kb + 1, lane, tb);
        work(ta, kb);
        load_ktile<T, H>(A, Kraw, kbuf, kb + 2 < kb1 ? kb + 2 : kb1 - 1, lane, ta);
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
        // logits in base 2: t = S * log2(e) / 8 (the scale is positive, so the
        // largest S gives the largest t)
        if (kb * 32 + 32 > M) {  // (uniform) the last, partial tile: keys past M do not count
#pragma unroll
          for (int r = 0; r < 16; ++r) S[r] = kb * 32 + crow(r, lane) < M ? S[r] : NEG;
        }
        float mx = S[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, S[r]);
        const float mnew = fmaxf(m[h], mx * 0.18033688011112042f);
        if (mnew != NEG) {
          float sum = 0.f;
#pragma unroll
          for (int r = 0; r < 16; ++r) sum += __builtin_amdgcn_exp2f(__builtin_fmaf(S[r], 0.18033688011112042f, -mnew));
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
    for (int i = tid; i < 2 * SEL_GB * NS * wst; i += SEL_NT) bits[i] = 0u;
    __syncthreads();
    // per (head, probe): max + log2(sum) over all tokens, so p = exp2(t - fin)
    if (tid < H * 32) {
      const int h = tid >> 5, c = tid & 31;
      float mm = NEG, ll = 0.f;
      for (int w = 0; w < SEL_NW; ++w) {
        const float2 st = stats[(w * H + h) * 32 + c];
        const float mn = fmaxf(mm, st.x);
        if (mn != NEG) {
          ll = ll * __builtin_amdgcn_exp2f(mm - mn) + st.y * __builtin_amdgcn_exp2f(st.x - mn);
          mm = mn;
        }
      }
      fin[tid] = mm + __builtin_amdgcn_logf(ll);
    }
    __syncthreads();

    // ---------------------------------------------------------------- pass 2: head-mean (or per-head) probabilities
    // K Q^T as in pass 1 (register r: token kb*32 + crow(r, lane), probe lane%32),
    // p = exp2(t - fin). Each wave transposes its 32 x 32 tile through its 4 KB of
    // the (not yet used) list region, so that every store writes 32 consecutive
    // tokens of one probe's row; rows are XOR-swizzled by the probe, which keeps
    // both the column writes and the row reads free of bank conflicts. (Rows of
    // probes past the group and tokens past M are written too: the scratch rows
    // hold Mp >= 32 * ceil(M / 32) values and the search reads only rows of the
    // group's probes and tokens below M.)
    lane = opaque(lane);
    col = lane & 31;
    float kcol[H];
#pragma unroll
    for (int h = 0; h < H; ++h) kcol[h] = fin[h * 32 + col];
    float* tb = reinterpret_cast<float*>(lds + CF::LISTS) + wave * SEL_LSTRIDE;  // [32 probes][32 tokens], swizzled
    const int rr = lane >> 5, kk = lane & 31;
    auto transpose_store = [&](const float (&v)[16], float* dst0, int rstride) {
#pragma unroll
      for (int r = 0; r < 16; ++r) tb[col * 32 + (crow(r, lane) ^ col)] = v[r];
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int pr = 2 * i + rr;
        dst0[pr * rstride + kk] = tb[pr * 32 + (kk ^ pr)];
      }
      __builtin_amdgcn_wave_barrier();  // the tile is read before the next one is written
    };
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
        if constexpr (PH) {
          // this head's probability is the score row (probe, head h)
          float pr[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) pr[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[r], 0.18033688011112042f, -kcol[h]));
          transpose_store(pr, scores + h * Mp + kb * 32, NS * Mp);
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[r] += __builtin_amdgcn_exp2f(__builtin_fmaf(S[r], 0.18033688011112042f, -kcol[h]));
        }
      }
      if constexpr (!PH) {
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] *= 1.f / H;
        transpose_store(acc, scores + kb * 32, Mp);
      }
    };
    over_key_tiles(score_tile);
    __syncthreads();  // the scores rows are complete and visible to the workgroup

    // ---------------------------------------------------------------- top-k per probe (and head), union per set
    // items (set, probe) in set order, a contiguous run per wave: a wave ORs the
    // masks of its probes of one set and adds them to the set's bitmap once
    tid = opaque(tid);
    lane = opaque(lane);
    {
      const int nit = nb * SEL_NP * NS, per = (nit + SEL_NW - 1) / SEL_NW;
      const int it1 = min(nit, (wave + 1) * per);
      uint64_t acc = 0ull;
      int cur = -1;
      for (int it = wave * per; it < it1; ++it) {
        const int set = it / SEL_NP, pr = it % SEL_NP;
        if (set != cur) {
          if constexpr (!BIG)  // (chunked rows mark their tokens directly)
            if (cur >= 0) add_to_bitmap(acc, M, bits + cur * wst, lane);
          acc = 0ull;
          cur = set;
        }
        // score row (probe, head): probe = block * NP + pr, head = set % NS
        const int srow = ((set / NS) * SEL_NP + pr) * NS + set % NS;
        if constexpr (!BIG) {
          unsigned u[SEL_MAXV];
          load_scores(scores, srow, Mp, M, lane, u);
          acc |= topk_mask(u, M, A.k, wlist, lane);
        } else {
          // each chunk's k largest, then the k largest of those (token order kept)
          int nc = 0;
          for (int c0 = 0; c0 < M; c0 += SEL_CHUNK) {
            unsigned u[SEL_MAXV];
            load_scores(scores, srow, Mp, M, lane, u, c0);
            const int n = min(SEL_CHUNK, M - c0);
            nc = append_tokens(topk_mask(u, n, A.k, wlist, lane), c0, n, cand, nc, lane);
          }
          nc = min(nc, SEL_LIST);
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
          unsigned v[SEL_CV];
#pragma unroll
          for (int j = 0; j < SEL_CV; ++j) {
            const int t = j * 64 + lane < nc ? cand[j * 64 + lane] : 0;
            const unsigned x = __builtin_amdgcn_raw_buffer_load_b32(sbuf, (srow * Mp + t) * 4, 0, 0);
            v[j] = j * 64 + lane < nc ? x : 0u;
          }
          mark_listed(topk_mask(v, nc, A.k, wlist, lane), cand, bits + set * wst, lane);
          __builtin_amdgcn_wave_barrier();  // the list is read before the next item writes it
        }
      }
      if constexpr (!BIG)
        if (cur >= 0) add_to_bitmap(acc, M, bits + cur * wst, lane);
    }
    __syncthreads();

    // ---------------------------------------------------------------- cap, compaction (one wave per set)
    tid = opaque(tid);
    lane = opaque(lane);
    for (int set = wave; set < nb * NS; set += SEL_NW) {
      const int blk = set / NS, hs = set % NS;
      unsigned* ub = bits + set * wst;
      int cnt = 0;
      for (int i = lane; i < nwords; i += 64) cnt += __popc(ub[i]);
      cnt = wave_sum(cnt);
      const unsigned* outbits = ub;
      if (BIG && cnt > A.cap) {
        // the same ranking over the union's members only (at most 8 k <= SEL_LIST),
        // listed in ascending token order, so equal scores keep their index order
        int base = 0;
        for (int w0 = 0; w0 < nwords; w0 += 64) {
          const int wi = w0 + lane;
          unsigned word = wi < nwords ? ub[wi] : 0u;
          const int c = __popc(word);
          const int incl = wave_incl_scan(c, lane);
          int off = base + incl - c;
          while (word) {
            const int b = __ffs(word) - 1;
            if (VDM_BOUND(off < SEL_LIST, BC_SELECT_CAND)) cand[off] = wi * 32 + b;
            ++off;
            word &= word - 1u;
          }
          base += __shfl(incl, 63);
        }
        const int nm = min(base, SEL_LIST);
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        unsigned v[SEL_CV];
#pragma unroll
        for (int j = 0; j < SEL_CV; ++j) {
          const bool in = j * 64 + lane < nm;
          const int t = in ? cand[j * 64 + lane] : 0;
          unsigned x = 0u;
#pragma unroll
          for (int q = 0; q < SEL_NP; ++q)
            x = max(x, __builtin_amdgcn_raw_buffer_load_b32(sbuf, ((((blk * SEL_NP + q) * NS + hs) * Mp) + t) * 4, 0, 0));
          v[j] = in ? x + 1u : 0u;
        }
        mark_listed(topk_mask(v, nm, A.cap, wlist, lane), cand, bits2 + set * wst, lane);
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        outbits = bits2 + set * wst;
      } else if (!BIG && cnt > A.cap) {
        // keep the cap tokens of largest max-over-probes score (members rank above non-members)
        unsigned u[SEL_MAXV];
        load_scores(scores, (blk * SEL_NP) * NS + hs, Mp, M, lane, u);
        for (int q = 1; q < SEL_NP; ++q) {
          const int voff = (((blk * SEL_NP + q) * NS + hs) * Mp + lane) * 4;
#pragma unroll
          for (int i = 0; i < SEL_MAXV; ++i)  // scores >= 0: bit order is float order
            u[i] = max(u[i], __builtin_amdgcn_raw_buffer_load_b32(sbuf, voff, i * 256, 0));
        }
        const int ln = opaque(lane);  // (the 64 indices are not hoisted out of the set loop)
#pragma unroll
        for (int i = 0; i < SEL_MAXV; ++i) {
          const int idx = i * 64 + ln;
          const bool member = idx < M && ((ub[idx >> 5] >> (idx & 31)) & 1u);
          u[i] = member ? u[i] + 1u : 0u;
        }
        add_to_bitmap(topk_mask(u, M, A.cap, wlist, lane), M, bits2 + set * wst, lane);
        outbits = bits2 + set * wst;
      }
      const int64_t row = (row0 + blk) * NS + hs;  // output row: [block][head] with per-head sets
#if VDM_DEBUG
      if (lane == 0) {
        const int NBs = (A.R + A.block) / A.block;
        const int64_t bid = blocks ? blocks[row0 + blk] : row0 + blk;
        (void)VDM_BOUND(bid >= 0 && bid < (int64_t)NBs * NBs * NBs, BC_SELECT_BLOCK);
      }
#endif
      int32_t* out = sel_idx + row * (int64_t)A.cap;
      int base = 0;
      for (int w0 = 0; w0 < nwords; w0 += 64) {
        const int wi = w0 + lane;
        unsigned word = wi < nwords ? outbits[wi] : 0u;
        const int c = __popc(word);
        const int incl = wave_incl_scan(c, lane);
        int off = base + incl - c;
        while (word) {
          const int b = __ffs(word) - 1;
          if (VDM_BOUND(off < A.cap, BC_SELECT_OUT)) out[off] = wi * 32 + b;
          ++off;
          word &= word - 1u;
        }
        base += __shfl(incl, 63);
      }
      for (int i = base + lane; i < A.cap; i += 64) out[i] = -1;
      if (lane == 0) {
        sel_cnt[row] = base;
        ucount[set] = base;
      }
    }
    __syncthreads();
    if (tid == 0 && stat_selected) {
      int64_t t = 0;
      for (int b = 0; b < nb * NS; ++b) t += ucount[b];
      atomicAdd((unsigned long long*)stat_selected, (unsigned long long)t);
    }
  }
}

template <typename T, int H, bool PH, bool BIG, bool RG = false>
static hipError_t run_select(const SelectArgs& a, hipStream_t s) {
  if (!RG && a.batch > 1 && a.grp_prefix) return run_select<T, H, PH, BIG, true>(a, s);
  const int lds = SelCfg<T, H, PH ? H : 1>::total(a.M);
  const void* fn = reinterpret_cast<const void*>(&select_kernel<T, H, PH, BIG, RG>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  int64_t grid = dev_info().cus;
  if (grid > SEL_GRID_MAX) grid = SEL_GRID_MAX;
  if (!a.d_n_blocks) {  // (a ragged batch counts on the device)
    const int64_t groups = (a.n_blocks + SEL_GB - 1) / SEL_GB;
    if (groups < grid) grid = groups;
  }
  if (grid < 1) return hipSuccess;
  hipLaunchKernelGGL((select_kernel<T, H, PH, BIG, RG>), dim3((unsigned)grid), dim3(SEL_NT), lds, s, a);
  return hipGetLastError();
}

size_t select_scratch_bytes(int M, int sets) {
  return (size_t)SEL_GRID_MAX * SEL_BQ * sets * sel_mpad(M) * sizeof(float);
}

int select_blocks_per_group() { return SEL_GB; }

int select_max_tokens(bool per_head) { return per_head ? SEL_MAX_M_PH : SEL_MAX_M; }

bool select_fits(int64_t M, int k, int cap, bool per_head) {
  if (M < 1 || M > select_max_tokens(per_head) || k < 1) return false;
  if (M <= SEL_CHUNK) return true;
  // chunk winners and the union's members fit a wave's list
  const int64_t chunks = (M + SEL_CHUNK - 1) / SEL_CHUNK;
  return (int64_t)k * chunks <= SEL_LIST && (cap >= SEL_NP * k || SEL_NP * k <= SEL_LIST);
}

template <typename T, int H, bool PH>
static hipError_t run_select_m(const SelectArgs& a, hipStream_t s) {
  return a.M > SEL_CHUNK ? run_select<T, H, PH, true>(a, s) : run_select<T, H, PH, false>(a, s);
}

hipError_t launch_select(int dtype, const SelectArgs& a, hipStream_t s) {
  if (!select_fits(a.M, a.k, a.cap, a.per_head != 0)) return hipErrorInvalidValue;
  if (dtype == VDM_BF16 && a.D == 256)
    return a.per_head ? run_select_m<bf16, 4, true>(a, s) : run_select_m<bf16, 4, false>(a, s);
  // (one head: its per-head set is the head-mean set)
  if (dtype == VDM_BF16) return run_select_m<bf16, 1, false>(a, s);
  return run_select_m<float, 1, false>(a, s);
}

VDM_DEBUG_READER(debug_take_select)

}  // namespace vdm
