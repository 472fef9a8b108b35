// The vecset decoder on gfx950: one kernel per tile of queries runs
//   Fourier embedding -> Q projection (MFMA) -> cross-attention over the token
//   set, K/V tiles staged in LDS, online softmax in registers (MFMA) ->
//   out-projection -> MLP with exact GELU and residual -> SDF head (MFMA)
//   -> + analytic prior.
// What it computes: the decoder of the FlashVDM pages (aipaper.cc summary,
// section 3: cross-attention from query points to the vecset yields the SDF;
// section 4.1 item 3: slim decoder without LayerNorm). Gathered mode restricts
// each tile to one block's token subset (section 4.1 item 2, Adaptive KV
// Selection; tiles of different blocks are packed into one launch).
//
// Layout of the work: a workgroup owns BQ queries. Wave w handles head
// w % H for query group w / H. S^T = K_h Q_h^T is computed with keys on MFMA rows
// and queries on columns, so every lane owns one query column: the softmax
// reductions over keys stay in-lane except one exchange between the two lane
// halves. P^T then feeds the P.V product straight from registers; the packed
// V^T tile stores tokens in the matching order (perm_key).
#include "vdm_device.hpp"

namespace vdm {

template <typename T_, int H_, int NW_, int QW_, int FC_>
struct DecCfg {
  typedef T_ T;
  static constexpr int H = H_, NW = NW_, QW = QW_, FC = FC_;
  static constexpr int D = 64 * H;
  static constexpr int NT = 64 * NW;
  static constexpr int G = NW / H;
  static constexpr int BQ = G * QW;
  static constexpr int QB = QW / 32;
  static constexpr int KT = 32;
  static constexpr int SZ = (int)sizeof(T);
  static constexpr int PAD = Pad<T>::v;
  static constexpr int DPAD = D + PAD;
  static constexpr int VPAD = KT + PAD;
  static constexpr int HPAD = FC + PAD;
  // attention stage: two K tiles [KT][DPAD] and two V^T tiles [D][VPAD]
  static constexpr int KBYTES = KT * DPAD * SZ;
  static constexpr int VBYTES = D * VPAD * SZ;
  static constexpr int ATT_END = 2 * (KBYTES + VBYTES);
  // epilogue: O [BQ][DPAD] (later the GELU chunk [BQ][HPAD]), a [BQ][DPAD], reduction
  static constexpr int OBUF = 0;
  static constexpr int ABUF = BQ * DPAD * SZ;
  static constexpr int RED = 2 * BQ * DPAD * SZ;
  static constexpr int EPI_END = RED + NW * BQ * 4;
  static constexpr int EMB_END = EmbedLds<T, BQ, D>::END;
  static constexpr int LDS = ATT_END > EPI_END ? (ATT_END > EMB_END ? ATT_END : EMB_END)
                                               : (EPI_END > EMB_END ? EPI_END : EMB_END);
  // epilogue tiling: wave w owns C tiles [w*TPW, (w+1)*TPW) of (D/32) x (BQ/32)
  static constexpr int CB = BQ / 32;
  static constexpr int TPW = (D / 32) * CB / NW;
  static constexpr int TPH = (FC / 32) * CB / NW;
  // global -> LDS staging: 16-byte chunks per thread per tile
  static constexpr int KCH = KT * D * SZ / 16;
  static constexpr int VCH = D * KT * SZ / 16;
  static constexpr int NCK = KCH / NT;
  static constexpr int NCV = VCH / NT;
  static constexpr int EPC = 16 / SZ;  // elements per chunk

  static_assert(NW % H == 0, "waves cover whole heads");
  static_assert(QW % 32 == 0, "query groups are whole MFMA columns");
  static_assert(BQ * HPAD * SZ <= ABUF, "GELU chunk fits where O was");
  static_assert(((D / 32) * CB) % NW == 0 && ((FC / 32) * CB) % NW == 0, "epilogue tiles split evenly");
  static_assert(CB % TPW == 0 && CB % TPH == 0, "a wave's epilogue tiles share one row block");
  static_assert(KCH % NT == 0 && VCH % NT == 0, "staging chunks split evenly");
  static_assert(LDS <= 160 * 1024, "fits gfx950 LDS");
};

// log2(e) / sqrt(64): softmax runs in base 2 on logits scaled once.
constexpr float SOFTMAX_SCALE_LOG2 = 0.18033688011112042f;

// Global -> registers: the K rows and V^T columns of 32-token tile kt.
// Dense: Kg = packed K [Mpad][D], Vg = packed V^T tiles [Mpad/32][D][32].
// Gathered: Kg, Vg = K, V [M][D]; token j of the tile is sel[32kt + j] (zero rows past nkeys).
// token ids of a selection are clamped into [0, M) so that no input can index past K/V
__device__ __forceinline__ int tok_clamp(int t, int M) { return t < 0 ? 0 : (t >= M ? M - 1 : t); }

template <typename C, bool GATHER>
__device__ __forceinline__ void load_kv_tile(const typename C::T* __restrict__ Kg, const typename C::T* __restrict__ Vg,
                                             const int32_t* sel, int nkeys, int M, int kt, int tid, uint4 (&rk)[C::NCK],
                                             uint4 (&rv)[C::NCV]) {
  constexpr int CPR = C::D / C::EPC;
  if constexpr (!GATHER) {
    const uint4* ks = reinterpret_cast<const uint4*>(Kg + (int64_t)kt * C::KT * C::D);
    const uint4* vs = reinterpret_cast<const uint4*>(Vg + (int64_t)kt * C::KT * C::D);
#pragma unroll
    for (int i = 0; i < C::NCK; ++i) rk[i] = ks[tid + i * C::NT];
#pragma unroll
    for (int i = 0; i < C::NCV; ++i) rv[i] = vs[tid + i * C::NT];
  } else {
#pragma unroll
    for (int i = 0; i < C::NCK; ++i) {
      const int c = tid + i * C::NT, j = kt * C::KT + c / CPR, e = (c % CPR) * C::EPC;
      rk[i] = j < nkeys ? *reinterpret_cast<const uint4*>(Kg + (int64_t)tok_clamp(sel[j], M) * C::D + e)
                        : uint4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < C::NCV; ++i) {
      const int c = tid + i * C::NT, j = kt * C::KT + c / CPR, e = (c % CPR) * C::EPC;
      rv[i] = j < nkeys ? *reinterpret_cast<const uint4*>(Vg + (int64_t)tok_clamp(sel[j], M) * C::D + e)
                        : uint4{0, 0, 0, 0};
    }
  }
}

// Registers -> LDS buffer `buf`: K tile [KT][DPAD]; V^T tile [D][VPAD] with the
// tile's tokens in perm_key order (dense: already packed; gathered: each
// thread's 16-byte run of one token's V row goes to column vpos of V^T).
template <typename C, bool GATHER>
__device__ __forceinline__ void store_kv_tile(char* lds, int buf, int tid, const int (&vpos)[C::NCV],
                                              const uint4 (&rk)[C::NCK], const uint4 (&rv)[C::NCV]) {
  using T = typename C::T;
  constexpr int CPR = C::D / C::EPC;
  T* Kb = reinterpret_cast<T*>(lds + buf * C::KBYTES);
  T* Vb = reinterpret_cast<T*>(lds + 2 * C::KBYTES + buf * C::VBYTES);
#pragma unroll
  for (int i = 0; i < C::NCK; ++i) {
    const int c = tid + i * C::NT;
    *reinterpret_cast<uint4*>(Kb + (c / CPR) * C::DPAD + (c % CPR) * C::EPC) = rk[i];
  }
  if constexpr (!GATHER) {
    constexpr int VCPR = C::KT / C::EPC;
#pragma unroll
    for (int i = 0; i < C::NCV; ++i) {
      const int c = tid + i * C::NT;
      *reinterpret_cast<uint4*>(Vb + (c / VCPR) * C::VPAD + (c % VCPR) * C::EPC) = rv[i];
    }
  } else {
#pragma unroll
    for (int i = 0; i < C::NCV; ++i) {
      const int e = ((tid + i * C::NT) % CPR) * C::EPC;
      const T* v = reinterpret_cast<const T*>(&rv[i]);
#pragma unroll
      for (int x = 0; x < C::EPC; ++x) Vb[(e + x) * C::VPAD + vpos[i]] = v[x];
    }
  }
}

template <typename C, bool GATHER>
__global__ __launch_bounds__(C::NT) void decode_kernel(DecodeArgs A) {
  extern __shared__ __align__(16) char lds[];
  using T = typename C::T;
  using MM = Mma<T>;
  using Frag = typename MM::frag;
  constexpr int KSTEPS_H = 64 / MM::KS;    // MFMA steps over one head's 64 columns
  constexpr int PSTEPS = C::KT / MM::KS;   // MFMA steps over one 32-token tile

  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int hw = wave % C::H, qg = wave / C::H;
  const int64_t nq = A.d_N ? (int64_t)*A.d_N : A.N;
  const int64_t n_tiles = A.items ? (A.d_n_items ? (int64_t)*A.d_n_items : A.n_tiles) : (nq + C::BQ - 1) / C::BQ;
  const T* __restrict__ Kg = (const T*)A.Kp;
  const T* __restrict__ Vg = (const T*)A.Vt;
  const T* __restrict__ Wo = (const T*)A.Wo;
  const T* __restrict__ W1 = (const T*)A.W1;
  const T* __restrict__ W2 = (const T*)A.W2;
  constexpr int CPR = C::D / C::EPC;  // 16-byte chunks per K / V row

  // gathered mode: where each staged V chunk lands inside the permuted tile
  int vpos[C::NCV];
#pragma unroll
  for (int i = 0; i < C::NCV; ++i) vpos[i] = key_pos<T>((tid + i * C::NT) / CPR);

  for (int64_t tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
    int64_t q0, q1;
    int row = -1;
    if (A.items) {
      const Item it = A.items[tile];
      q0 = it.q0;
      q1 = it.q1;
      row = it.row;
    } else {
      q0 = tile * C::BQ;
      q1 = q0 + C::BQ < nq ? q0 + C::BQ : nq;
    }

    // ---------------------------------------------------------------- Q = Wq e(p)
    embed_qproj<T, C::BQ, C::D, C::NT>(A.qs, q0, q1, (const T*)A.Wq, lds, tid);
    Frag qf[C::QB][KSTEPS_H];
    {
      const T* Qs = reinterpret_cast<const T*>(lds + EmbedLds<T, C::BQ, C::D>::QS);
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb)
#pragma unroll
        for (int ks = 0; ks < KSTEPS_H; ++ks)
          qf[qb][ks] = load_frag<T>(Qs + (qg * C::QW + 32 * qb) * C::DPAD + 64 * hw + ks * MM::KS, C::DPAD, lane);
    }
    __syncthreads();

    // ---------------------------------------------------------------- attention
    // selected-token count clamped to [0, cap] (a row never reads past its cap entries)
    const int nkeys = GATHER ? min(max(A.sel_cnt[row], 0), A.cap) : A.M;
    const int32_t* sel = GATHER ? A.sel_idx + (int64_t)row * A.cap : nullptr;
    const int nkt = (nkeys + C::KT - 1) / C::KT;

    uint4 rk[C::NCK], rv[C::NCV];

    f32x16 O[2][C::QB];
    float m_run[C::QB], l_run[C::QB];
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) {
      O[0][qb] = zero16();
      O[1][qb] = zero16();
      m_run[qb] = -__builtin_inff();
      l_run[qb] = 0.f;
    }

    load_kv_tile<C, GATHER>(Kg, Vg, sel, nkeys, A.M, 0, tid, rk, rv);
    store_kv_tile<C, GATHER>(lds, 0, tid, vpos, rk, rv);
    __syncthreads();
    for (int kt = 0; kt < nkt; ++kt) {
      // prefetch the next tile (the last iteration reloads its own tile: always in bounds)
      const int knext = kt + 1 < nkt ? kt + 1 : kt;
      load_kv_tile<C, GATHER>(Kg, Vg, sel, nkeys, A.M, knext, tid, rk, rv);
      const T* Kb = reinterpret_cast<const T*>(lds + (kt & 1) * C::KBYTES);
      const T* Vb = reinterpret_cast<const T*>(lds + 2 * C::KBYTES + (kt & 1) * C::VBYTES);

      f32x16 S[C::QB];
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb) S[qb] = zero16();
#pragma unroll
      for (int ks = 0; ks < KSTEPS_H; ++ks) {
        const Frag kf = load_frag<T>(Kb + 64 * hw + ks * MM::KS, C::DPAD, lane);
#pragma unroll
        for (int qb = 0; qb < C::QB; ++qb) S[qb] = MM::mma(kf, qf[qb][ks], S[qb]);
      }

      Frag pf[C::QB][PSTEPS];
      const bool ragged = (kt + 1) * C::KT > nkeys;
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb) {
        float t[16];
        float mx = -__builtin_inff();
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          t[r] = S[qb][r] * SOFTMAX_SCALE_LOG2;
          if (ragged && kt * C::KT + crow(r, lane) >= nkeys) t[r] = -__builtin_inff();
          mx = fmaxf(mx, t[r]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mnew = fmaxf(m_run[qb], mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - mnew);
        float lsum = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          t[r] = __builtin_amdgcn_exp2f(t[r] - mnew);
          lsum += t[r];
        }
        l_run[qb] = l_run[qb] * alpha + lsum;
        m_run[qb] = mnew;
        O[0][qb] *= alpha;
        O[1][qb] *= alpha;
#pragma unroll
        for (int ps = 0; ps < PSTEPS; ++ps) {
          if constexpr (MM::KW == 1) {
            pf[qb][ps] = t[ps];
          } else {
            Frag f;
#pragma unroll
            for (int v = 0; v < MM::KW; ++v) f[v] = to_t<T>(t[MM::KW * ps + v]);
            pf[qb][ps] = f;
          }
        }
      }
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int ps = 0; ps < PSTEPS; ++ps) {
          const Frag vf = load_frag<T>(Vb + (64 * hw + 32 * db) * C::VPAD + ps * MM::KS, C::VPAD, lane);
#pragma unroll
          for (int qb = 0; qb < C::QB; ++qb) O[db][qb] = MM::mma(vf, pf[qb][ps], O[db][qb]);
        }
      // the other buffer was last read before the previous barrier
      store_kv_tile<C, GATHER>(lds, (kt + 1) & 1, tid, vpos, rk, rv);
      __syncthreads();
    }

    // ---------------------------------------------------------------- o = softmax-weighted V
    T* Ob = reinterpret_cast<T*>(lds + C::OBUF);
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) {
      const float inv = 1.f / (l_run[qb] + __shfl_xor(l_run[qb], 32));
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        O[db][qb] *= inv;
        store_ct<T>(Ob + (qg * C::QW + 32 * qb) * C::DPAD + 64 * hw + 32 * db, C::DPAD, O[db][qb], lane);
      }
    }
    __syncthreads();

    // ---------------------------------------------------------------- a = Wo o  (kept in fp32 as y)
    const int rb = (wave * C::TPW) / C::CB;  // this wave's 32-row block of D
    f32x16 Y[C::TPW];
#pragma unroll
    for (int i = 0; i < C::TPW; ++i) Y[i] = zero16();
    for (int ks = 0; ks < C::D / MM::KS; ++ks) {
      const Frag af = load_frag<T>(Wo + (32 * rb) * C::D + ks * MM::KS, C::D, lane);
#pragma unroll
      for (int i = 0; i < C::TPW; ++i) {
        const int cb = (wave * C::TPW + i) % C::CB;
        Y[i] = MM::mma(af, load_frag<T>(Ob + (32 * cb) * C::DPAD + ks * MM::KS, C::DPAD, lane), Y[i]);
      }
    }
    T* Ab = reinterpret_cast<T*>(lds + C::ABUF);
#pragma unroll
    for (int i = 0; i < C::TPW; ++i) {
      const int cb = (wave * C::TPW + i) % C::CB;
      store_ct<T>(Ab + (32 * cb) * C::DPAD + 32 * rb, C::DPAD, Y[i], lane);
    }
    __syncthreads();

    // ---------------------------------------------------------------- y = a + W2 GELU(W1 a)
    T* Hb = reinterpret_cast<T*>(lds + C::OBUF);
    const int rbh = (wave * C::TPH) / C::CB;
    for (int f0 = 0; f0 < A.F; f0 += C::FC) {
      f32x16 Hc[C::TPH];
#pragma unroll
      for (int j = 0; j < C::TPH; ++j) Hc[j] = zero16();
      for (int ks = 0; ks < C::D / MM::KS; ++ks) {
        const Frag af = load_frag<T>(W1 + (int64_t)(f0 + 32 * rbh) * C::D + ks * MM::KS, C::D, lane);
#pragma unroll
        for (int j = 0; j < C::TPH; ++j) {
          const int cb = (wave * C::TPH + j) % C::CB;
          Hc[j] = MM::mma(af, load_frag<T>(Ab + (32 * cb) * C::DPAD + ks * MM::KS, C::DPAD, lane), Hc[j]);
        }
      }
#pragma unroll
      for (int j = 0; j < C::TPH; ++j) {
        const int cb = (wave * C::TPH + j) % C::CB;
#pragma unroll
        for (int r = 0; r < 16; ++r) Hc[j][r] = gelu(Hc[j][r]);
        store_ct<T>(Hb + (32 * cb) * C::HPAD + 32 * rbh, C::HPAD, Hc[j], lane);
      }
      __syncthreads();
      for (int ks = 0; ks < C::FC / MM::KS; ++ks) {
        const Frag af = load_frag<T>(W2 + (int64_t)(32 * rb) * A.F + f0 + ks * MM::KS, A.F, lane);
#pragma unroll
        for (int i = 0; i < C::TPW; ++i) {
          const int cb = (wave * C::TPW + i) % C::CB;
          Y[i] = MM::mma(af, load_frag<T>(Hb + (32 * cb) * C::HPAD + ks * MM::KS, C::HPAD, lane), Y[i]);
        }
      }
      __syncthreads();
    }

    // ---------------------------------------------------------------- net = w_head . y, SDF
    float* red = reinterpret_cast<float*>(lds + C::RED);
    {
      float w[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) w[r] = A.w_head[32 * rb + crow(r, lane)];
      // this wave's column blocks are cb0 .. cb0 + TPW - 1; the rest get zeros
      const int cb0 = (wave * C::TPW) % C::CB;
#pragma unroll
      for (int i = 0; i < C::TPW; ++i) {
        float s = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) s += w[r] * Y[i][r];
        s += __shfl_xor(s, 32);
        if (lane < 32) red[wave * C::BQ + 32 * (cb0 + i) + lane] = s;
      }
      for (int cb = 0; cb < C::CB; ++cb)
        if ((cb < cb0 || cb >= cb0 + C::TPW) && lane < 32) red[wave * C::BQ + 32 * cb + lane] = 0.f;
    }
    __syncthreads();
    for (int t = tid; t < C::BQ; t += C::NT) {
      const int64_t q = q0 + t;
      if (q < q1) {
        float net = 0.f;
#pragma unroll
        for (int w = 0; w < C::NW; ++w) net += red[w * C::BQ + t];
        const Coords p = query_coords(A.qs, q);
        const float sdf = analytic_sdf(p, A.prims) + A.net_scale * net;
        int64_t o = q;
        if (A.scatter) o = A.qs.mode == 1 ? q : (int64_t)A.qs.list[q];
        A.out[o] = sdf;
      }
    }
    __syncthreads();
  }
}

typedef DecCfg<bf16, 4, 8, 64, 128> CfgB256;
typedef DecCfg<bf16, 1, 4, 32, 64> CfgB64;
typedef DecCfg<float, 1, 4, 32, 64> CfgF64;

template <typename C, bool GATHER>
static hipError_t run(const DecodeArgs& a, hipStream_t s) {
  static bool attr = false;
  const void* fn = reinterpret_cast<const void*>(&decode_kernel<C, GATHER>);
  if (!attr) {
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
    if (e != hipSuccess) return e;
    attr = true;
  }
  int per_cu = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_kernel<C, GATHER>, C::NT, C::LDS);
  if (e != hipSuccess) return e;
  if (per_cu < 1) per_cu = 1;
  int64_t grid = (int64_t)dev_info().cus * per_cu;
  if (!a.d_N && !a.d_n_items) {
    const int64_t host_tiles = a.items ? a.n_tiles : (a.N + C::BQ - 1) / C::BQ;
    if (host_tiles < grid) grid = host_tiles;
  }
  if (grid < 1) return hipSuccess;
  hipLaunchKernelGGL((decode_kernel<C, GATHER>), dim3((unsigned)grid), dim3(C::NT), C::LDS, s, a);
  return hipGetLastError();
}

hipError_t launch_decode(int dtype, int D, bool gathered, const DecodeArgs& a, hipStream_t s) {
  if (dtype == VDM_BF16 && D == 256) return gathered ? run<CfgB256, true>(a, s) : run<CfgB256, false>(a, s);
  if (dtype == VDM_BF16 && D == 64) return gathered ? run<CfgB64, true>(a, s) : run<CfgB64, false>(a, s);
  return gathered ? run<CfgF64, true>(a, s) : run<CfgF64, false>(a, s);
}

int decode_tile_queries(int dtype, int D) {
  if (dtype == VDM_BF16 && D == 256) return CfgB256::BQ;
  if (dtype == VDM_BF16) return CfgB64::BQ;
  return CfgF64::BQ;
}

int decode_f_chunk(int dtype, int D) {
  if (dtype == VDM_BF16 && D == 256) return CfgB256::FC;
  if (dtype == VDM_BF16) return CfgB64::FC;
  return CfgF64::FC;
}

}  // namespace vdm
