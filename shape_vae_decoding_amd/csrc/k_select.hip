// Adaptive KV Selection on gfx950 (FlashVDM summary, section 4.1 item 2: per
// sub-volume, a few probe queries attend to all latent tokens and the highest
// scoring tokens become the sub-volume's key/value set; techwalker article,
// part 5, describes the same probe-then-reuse scheme).
//
// One workgroup per block: the block's 8 corner probes are embedded and
// projected (same device routine as the decoder), then
//   pass 1: per (probe, head) softmax max and sum over all tokens (MFMA logits),
//   pass 2: score_j = mean over heads of the softmax probability, kept in LDS,
//   top-k per probe by an exact 4-digit radix select on the float bits
//   (equal scores: lower token index first), union in an LDS bitmap, optional
//   cap by max-over-probes score, ascending compaction.
// Each wave covers a quarter of the tokens for all heads; the per-wave partial
// softmax statistics are merged in a fixed order, so results are reproducible.
#include "vdm_device.hpp"

namespace vdm {

constexpr int SEL_NT = 256;
constexpr int SEL_NW = SEL_NT / 64;
constexpr int SEL_NP = 8;   // probes per block
constexpr int SEL_BQ = 32;  // probe columns of the MFMA tile (8 used)

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o);
    if (lane >= o) v += u;
  }
  return v;
}

// Mark in `bits` the k largest of the M values getu(i) (unsigned order; equal
// values: lower index first). One wave; `hist` is 256 ints of this wave's LDS.
template <typename GetU>
__device__ void topk_mark(GetU getu, int M, int k, int* hist, unsigned* bits, int lane) {
  unsigned prefix = 0, pmask = 0;
  int need = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = lane; i < 256; i += 64) hist[i] = 0;
    wave_sync();
    for (int i = lane; i < M; i += 64) {
      const unsigned u = getu(i);
      if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & 255], 1);
    }
    wave_sync();
    // lane holds bins 255-4l .. 252-4l (descending digit order)
    const int c0 = hist[255 - 4 * lane], c1 = hist[254 - 4 * lane], c2 = hist[253 - 4 * lane],
              c3 = hist[252 - 4 * lane];
    const int tot = c0 + c1 + c2 + c3;
    const int incl = wave_incl_scan(tot, lane);
    const int excl = incl - tot;
    const bool mine = excl < need && need <= incl;
    int digit = 0, before = 0;
    if (mine) {
      int c = excl;
      if (c + c0 >= need) {
        digit = 255 - 4 * lane;
      } else if ((c += c0) + c1 >= need) {
        digit = 254 - 4 * lane;
      } else if ((c += c1) + c2 >= need) {
        digit = 253 - 4 * lane;
      } else {
        c += c2;
        digit = 252 - 4 * lane;
      }
      before = c;
    }
    const unsigned long long bal = __ballot(mine);
    const int src = __ffsll((long long)bal) - 1;
    digit = __shfl(digit, src);
    before = __shfl(before, src);
    need -= before;
    prefix |= (unsigned)digit << shift;
    pmask |= 255u << shift;
    wave_sync();
  }
  // prefix is now the k-th largest value; `need` of its copies are taken, lowest index first
  int taken = 0;
  for (int base = 0; base < M; base += 64) {
    const int i = base + lane;
    const unsigned u = i < M ? getu(i) : 0u;
    const bool eq = i < M && u == prefix;
    const bool gt = i < M && u > prefix;
    const unsigned long long be = __ballot(eq);
    const int rank = __popcll(be & ((1ull << lane) - 1ull));
    if (gt || (eq && taken + rank < need)) atomicOr(&bits[i >> 5], 1u << (i & 31));
    taken += __popcll(be);
  }
  wave_sync();
}

template <typename T, int H>
struct SelCfg {
  static constexpr int D = 64 * H;
  static constexpr int EMB_END = EmbedLds<T, SEL_BQ, D>::END;
  __host__ __device__ static int base(int M) {
    const int s = SEL_NP * M * 4;
    return ((s > EMB_END ? s : EMB_END) + 15) & ~15;
  }
  __host__ __device__ static int total(int M) {
    const int words = (M + 31) / 32;
    return base(M) + SEL_NW * H * 32 * 8 + SEL_NW * 256 * 4 + 2 * words * 4 + 16;
  }
};

template <typename T, int H>
__global__ __launch_bounds__(SEL_NT) void select_kernel(SelectArgs A) {
  extern __shared__ __align__(16) char lds[];
  using MM = Mma<T>;
  using Frag = typename MM::frag;
  using L = EmbedLds<T, SEL_BQ, 64 * H>;
  constexpr int D = 64 * H, KS_H = 64 / MM::KS;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int M = A.M;
  const int nwords = (M + 31) / 32;
  const int lbase = SelCfg<T, H>::base(M);
  float* scores = reinterpret_cast<float*>(lds);                              // [8][M]
  float2* stats = reinterpret_cast<float2*>(lds + lbase);                     // [NW][H][32]
  int* hist = reinterpret_cast<int*>(lds + lbase + SEL_NW * H * 32 * 8);      // [NW][256]
  unsigned* bits = reinterpret_cast<unsigned*>(hist + SEL_NW * 256);          // [nwords]
  unsigned* bits2 = bits + nwords;                                            // [nwords]
  const int64_t nblk = A.d_n_blocks ? (int64_t)*A.d_n_blocks : A.n_blocks;
  const T* __restrict__ K = (const T*)A.K;
  QuerySrc qs;
  qs.mode = 3;
  qs.R = A.R;
  qs.xyz = nullptr;
  qs.list = A.blocks;
  qs.block = A.block;
  const int nkb = (M + 31) / 32;
  const int per = (nkb + SEL_NW - 1) / SEL_NW;
  const int kb0 = wave * per, kb1 = min(nkb, kb0 + per);
  const int col = lane & 31;
  const float NEG = -__builtin_inff();

  for (int64_t row = blockIdx.x; row < nblk; row += gridDim.x) {
    embed_qproj<T, SEL_BQ, D, SEL_NT>(qs, row * SEL_NP, row * SEL_NP + SEL_NP, (const T*)A.Wq, lds, tid);
    Frag qf[H][KS_H];
    {
      const T* Qs = reinterpret_cast<const T*>(lds + L::QS);
#pragma unroll
      for (int h = 0; h < H; ++h)
#pragma unroll
        for (int ks = 0; ks < KS_H; ++ks) qf[h][ks] = load_frag<T>(Qs + 64 * h + ks * MM::KS, L::DPAD, lane);
    }
    __syncthreads();
    for (int i = tid; i < 2 * nwords; i += SEL_NT) bits[i] = 0u;

    // ---------------------------------------------------------------- pass 1: softmax statistics
    float m[H], l[H];
#pragma unroll
    for (int h = 0; h < H; ++h) {
      m[h] = NEG;
      l[h] = 0.f;
    }
    for (int kb = kb0; kb < kb1; ++kb) {
      const int key = min(kb * 32 + (lane & 31), M - 1);
      const T* krow = K + (int64_t)key * D + MM::KW * (lane >> 5);
#pragma unroll
      for (int h = 0; h < H; ++h) {
        f32x16 S = zero16();
#pragma unroll
        for (int ks = 0; ks < KS_H; ++ks)
          S = MM::mma(*reinterpret_cast<const Frag*>(krow + 64 * h + ks * MM::KS), qf[h][ks], S);
        float mx = NEG;
        float t[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          t[r] = kb * 32 + crow(r, lane) < M ? S[r] * 0.18033688011112042f : NEG;
          mx = fmaxf(mx, t[r]);
        }
        const float mnew = fmaxf(m[h], mx);
        if (mnew != NEG) {
          float s = 0.f;
#pragma unroll
          for (int r = 0; r < 16; ++r) s += __builtin_amdgcn_exp2f(t[r] - mnew);
          l[h] = l[h] * __builtin_amdgcn_exp2f(m[h] - mnew) + s;
          m[h] = mnew;
        }
      }
    }
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
    for (int kb = kb0; kb < kb1; ++kb) {
      const int key = min(kb * 32 + (lane & 31), M - 1);
      const T* krow = K + (int64_t)key * D + MM::KW * (lane >> 5);
      float acc[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
      for (int h = 0; h < H; ++h) {
        f32x16 S = zero16();
#pragma unroll
        for (int ks = 0; ks < KS_H; ++ks)
          S = MM::mma(*reinterpret_cast<const Frag*>(krow + 64 * h + ks * MM::KS), qf[h][ks], S);
#pragma unroll
        for (int r = 0; r < 16; ++r)
          acc[r] += __builtin_amdgcn_exp2f(S[r] * 0.18033688011112042f - mf[h]) * linv[h];
      }
      if (col < SEL_NP) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = kb * 32 + crow(r, lane);
          if (j < M) scores[col * M + j] = acc[r] * (1.f / H);
        }
      }
    }
    __syncthreads();

    // ---------------------------------------------------------------- top-k per probe, union
    for (int p = wave; p < SEL_NP; p += SEL_NW) {
      const float* sc = scores + p * M;
      topk_mark([&](int i) { return __float_as_uint(sc[i]); }, M, A.k, hist + wave * 256, bits, lane);
    }
    __syncthreads();
    int cnt = 0;
    for (int i = lane; i < nwords; i += 64) cnt += __popc(bits[i]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) cnt += __shfl_xor(cnt, o);
    unsigned* outbits = bits;
    if (cnt > A.cap) {
      // keep the cap tokens of largest max-over-probes score (members rank above non-members)
      if (wave == 0) {
        auto getu = [&](int i) -> unsigned {
          if (!((bits[i >> 5] >> (i & 31)) & 1u)) return 0u;
          float mx = scores[i];
          for (int p = 1; p < SEL_NP; ++p) mx = fmaxf(mx, scores[p * M + i]);
          return __float_as_uint(mx) + 1u;
        };
        topk_mark(getu, M, A.cap, hist, bits2, lane);
      }
      outbits = bits2;
      __syncthreads();
    }

    // ---------------------------------------------------------------- ascending compaction
    if (wave == 0) {
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
        if (A.stat_selected) atomicAdd((unsigned long long*)A.stat_selected, (unsigned long long)base);
      }
    }
    __syncthreads();
  }
}

template <typename T, int H>
static hipError_t run_select(const SelectArgs& a, hipStream_t s) {
  const int lds = SelCfg<T, H>::total(a.M);
  const void* fn = reinterpret_cast<const void*>(&select_kernel<T, H>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  int per_cu = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, select_kernel<T, H>, SEL_NT, lds);
  if (e != hipSuccess) return e;
  if (per_cu < 1) per_cu = 1;
  int64_t grid = (int64_t)dev_info().cus * per_cu;
  if (!a.d_n_blocks && a.n_blocks < grid) grid = a.n_blocks;
  if (grid < 1) return hipSuccess;
  hipLaunchKernelGGL((select_kernel<T, H>), dim3((unsigned)grid), dim3(SEL_NT), lds, s, a);
  return hipGetLastError();
}

size_t select_lds_bytes(int dtype, int D, int M) {
  if (dtype == VDM_BF16) return D == 256 ? SelCfg<bf16, 4>::total(M) : SelCfg<bf16, 1>::total(M);
  return SelCfg<float, 1>::total(M);
}

hipError_t launch_select(int dtype, const SelectArgs& a, hipStream_t s) {
  if (dtype == VDM_BF16) return a.D == 256 ? run_select<bf16, 4>(a, s) : run_select<bf16, 1>(a, s);
  return run_select<float, 1>(a, s);
}

}  // namespace vdm
