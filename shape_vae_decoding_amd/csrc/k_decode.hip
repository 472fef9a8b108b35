// The vecset decoder on gfx950: one workgroup per tile of queries runs
//   Fourier embedding -> Q projection (MFMA) -> cross-attention over the token
//   set (MFMA, softmax in registers) -> out-projection -> MLP with exact GELU
//   and residual -> SDF head (MFMA) -> + analytic prior.
// What it computes: the decoder of the FlashVDM pages (aipaper.cc summary,
// section 3: cross-attention from query points to the vecset yields the SDF;
// section 4.1 item 3: slim decoder without LayerNorm). Gathered mode restricts
// each tile to one block's token subset (section 4.1 item 2, Adaptive KV
// Selection; tiles of different blocks are packed into one launch).
//
// Work layout: wave w handles head w % H for query group w / H. S^T = K_h Q_h^T
// puts keys on MFMA rows and queries on columns, so a lane owns one query
// column and the P.V product takes P^T straight from the C registers; the
// packed V^T operand stores tokens in the matching order (perm_key).
//
// Softmax with a fixed shift: queries are scaled by log2(e)/8 before their
// rounding, so S holds base-2 logits t. For query q and head h,
//   B = ||q_h|| * max_j ||k_hj||  >=  |t_j| for every token (Cauchy-Schwarz),
// and p_j = exp2(t_j + nb), o = sum_j p_j v_j / sum_j p_j. When every query of
// the wave has B <= 64, nb = 0 (p_j in [2^-64, 2^64]: no overflow, no
// underflow). Otherwise the wave first takes each query's true maximum logit
// t_max over the tokens (a pass of the same S products, so the same values) and
// uses nb = 64 - t_max: p_j <= 2^64 and the largest p_j is 2^64, so the row sum
// cannot vanish however loose B is (a key with a large component that no query
// sees, e.g. outside the span of the head's Wq rows, makes B large without
// raising any logit). The softmax is shift-invariant, so both equal the
// max-subtracted definition in exact arithmetic. No running maximum in the main
// pass, no rescaling of O. The row sum is accumulated from the bf16-rounded p_j
// (dot2 with ones), the same values the P.V product uses.
//
// Dense mode: each wave streams its head's pre-packed K and V^T operand runs
// straight from L2 into registers (no LDS, no barriers in the token loop), in a
// software pipeline that overlaps the loads, the P.V and S MFMAs and the softmax;
// for bf16 the two waves of a head that share a SIMD (its two query groups) run
// that loop under different instruction schedules (dense_attention_2phase).
// Gathered mode reads the selected tokens' rows into LDS stages (two K, three V;
// V read transposed), one barrier per 32-token tile.
// The epilogue streams each weight row once per workgroup from L2 through a
// 4-deep register prefetch ring that runs through the chain of products (Wo,
// then W1 and W2 per hidden chunk): each product starts with its first weights
// already requested, across the barrier before it.
#include "vdm_device.hpp"

namespace vdm {

// segments of the bf16 GELU table (see gelu_lookup)
constexpr int GELU_SEGS = 2048;
constexpr float GELU_LIM = 8.f;
constexpr float GELU_SCALE = GELU_SEGS / (2.f * GELU_LIM);

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
  static constexpr int KSTEPS = 64 / Mma<T>::KS;   // MFMA steps over one head's 64 columns
  static constexpr int PSTEPS = KT / Mma<T>::KS;   // MFMA steps over one 32-token tile
  // per-lane operand run of one (tile, head): 32 elements of K and 32 of V^T
  static constexpr int RUN_U4 = 32 * SZ / 16;
  // gathered-mode staging: two K tiles [KT][DPAD] and two (three for the
  // software-pipelined 16-bit path) V tiles, row-major
  // [KT][VROW] for 16-bit types (read transposed by ds_read_b64_tr_b16; rows of
  // D + 32 elements put the 4 rows of one read 16 banks apart) or V^T [D][VPAD]
  static constexpr bool TR_V = SZ == 2;
  static constexpr int VROW = D + 32;
  static constexpr int KBYTES = KT * DPAD * SZ;
  static constexpr int VBYTES = TR_V ? KT * VROW * SZ : D * VPAD * SZ;
  static constexpr int ATT_END = 2 * KBYTES + (TR_V ? 3 : 2) * VBYTES;
  // epilogue: O [BQ][DPAD] (later the GELU chunk [BQ][HPAD]), a [BQ][DPAD], reduction
  static constexpr int OBUF = 0;
  static constexpr int ABUF = BQ * DPAD * SZ;
  static constexpr int RED = 2 * BQ * DPAD * SZ;
  static constexpr int EPI_END = RED + NW * BQ * 4;
  static constexpr int EMB_END = EmbedLds<T, BQ, D>::END;
  static constexpr int LDS_PRE = EPI_END > EMB_END ? EPI_END : EMB_END;
  static constexpr int LDS_MAIN = LDS_PRE > ATT_END ? LDS_PRE : ATT_END;
  // bf16: GELU table (value, slope) per segment, resident for the whole kernel
  static constexpr bool GELU_TABLE = sizeof(T) == 2;
  // bf16: Wo, W1, W2 arrive fragment-packed (one contiguous 1 KB per MFMA step)
  static constexpr bool PACKED_W = sizeof(T) == 2;
  static constexpr int GTAB = LDS_MAIN;
  static constexpr int LDS = LDS_MAIN + (GELU_TABLE ? GELU_SEGS * 8 : 0);
  // epilogue tiling: wave w owns C tiles [w*TPW, (w+1)*TPW) of (D/32) x (BQ/32), rb-major:
  // one row block of weights (loaded once per workgroup) for TPW column blocks
  static constexpr int CB = BQ / 32;
  static constexpr int TPW = (D / 32) * CB / NW;
  static constexpr int TPH = (FC / 32) * CB / NW;
  // a wave owns RPW row blocks x CPW column blocks of the D x BQ outputs (RPH x CPH
  // of an FC x BQ hidden chunk): whole rows of column blocks when it has that many
  static constexpr int RPW = TPW >= CB ? TPW / CB : 1, CPW = TPW >= CB ? CB : TPW;
  static constexpr int RPH = TPH >= CB ? TPH / CB : 1, CPH = TPH >= CB ? CB : TPH;
  // staging: 16-byte chunks per thread per tile (K and V each)
  static constexpr int KCH = KT * D * SZ / 16;
  static constexpr int NCK = KCH / NT;
  static constexpr int EPC = 16 / SZ;
  // explicit MFMA / softmax interleaving in the token loop (bf16, 2+ query blocks)
  static constexpr bool SCHED_ATT = SZ == 2 && QB >= 2;

  static_assert(NW % H == 0, "waves cover whole heads");
  static_assert(QW % 32 == 0, "query groups are whole MFMA columns");
  static_assert(BQ * HPAD * SZ <= ABUF, "GELU chunk fits where O was");
  static_assert(((D / 32) * CB) % NW == 0 && ((FC / 32) * CB) % NW == 0, "epilogue tiles split evenly");
  static_assert(TPW >= CB ? TPW % CB == 0 : CB % TPW == 0, "output tiles split evenly");
  static_assert(TPH >= CB ? TPH % CB == 0 : CB % TPH == 0, "hidden tiles split evenly");
  static_assert(KCH % NT == 0, "staging chunks split evenly");
  static_assert(LDS <= 160 * 1024, "fits gfx950 LDS");
};

// GELU by table for bf16 decoders: GELU_SEGS linear segments over [-GELU_LIM, GELU_LIM]
// (width 1/128), each stored as (GELU(x_i), GELU(x_{i+1}) - GELU(x_i)); interpolation
// error <= h^2/8 max|GELU''| < 7e-6, far below the bf16 rounding of the hidden
// activations. The first segment is flat at GELU(-8) (|GELU| < 6e-15 there). Past
// the range the end segments extrapolate: x > 8 continues the last segment, whose
// slope is 1 to within 1e-14, so the value is x to within 1e-14 (as GELU is);
// x < -8 stays at GELU(-8). NaN gives NaN; -inf gives NaN.

__device__ __forceinline__ void gelu_table_fill(float2* tab, int tid, int nt) {
  for (int i = tid; i < GELU_SEGS; i += nt) {
    const float x0 = -GELU_LIM + (float)i / GELU_SCALE, x1 = -GELU_LIM + (float)(i + 1) / GELU_SCALE;
    const float g0 = gelu(x0);
    tab[i] = make_float2(g0, i == 0 ? 0.f : gelu(x1) - g0);
  }
}

// GELU of the 16 values of one C tile, branch-free: the segment index is clamped
// into the table, the offset within it is not (so the end segments extrapolate).
// All 16 table reads are issued before the first is used, so their LDS latency
// overlaps.
template <typename C>
__device__ __forceinline__ void gelu_tile(f32x16& h, const float2* tab) {
  if constexpr (C::GELU_TABLE) {
    float t[16];
    int seg[16];
    float2 e[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      t[r] = __builtin_fmaf(h[r], GELU_SCALE, GELU_LIM * GELU_SCALE);
      seg[r] = (int)__builtin_amdgcn_fmed3f(t[r], 0.f, (float)GELU_SEGS - 0.5f);
      e[r] = tab[seg[r]];
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) h[r] = __builtin_fmaf(e[r].y, t[r] - (float)seg[r], e[r].x);
  } else {
#pragma unroll
    for (int r = 0; r < 16; ++r) h[r] = gelu(h[r]);
  }
}

// log2(e) / sqrt(64): logits are scaled once into base 2.
constexpr float SOFTMAX_SCALE_LOG2 = 0.18033688011112042f;

// token ids of a selection are clamped into [0, M) so that no input can index past K/V
__device__ __forceinline__ int tok_clamp(int t, int M) {
  (void)VDM_BOUND(t >= 0 && t < M, BC_DECODE_TOKEN);
  return t < 0 ? 0 : (t >= M ? M - 1 : t);
}

// Packed K/V operands are read with buffer loads: the tile/head base is a scalar
// offset, the lane's run a fixed vector offset; reads past the buffer's size
// return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_of(const void* p, int64_t bytes) {
  constexpr int GFX9_RAW_BUFFER = 0x00020000;  // descriptor word 3: raw (untyped) buffer
  const int n = bytes < 0x7fffffff ? (int)bytes : 0x7fffffff;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, n, GFX9_RAW_BUFFER);
}

// One lane's operand run (32 elements) of packed tile `kt`, head h: chunk i of
// all lanes is a contiguous 1 KB, so each load reads 1 KB without gaps.
template <typename C>
__device__ __forceinline__ void load_run(__amdgpu_buffer_rsrc_t buf, int kt, int h, int lane,
                                         uint4 (&r)[C::RUN_U4]) {
  const int soff = (kt * C::H + h) * 64 * 32 * C::SZ;
  const int voff = lane * 16;
#pragma unroll
  for (int i = 0; i < C::RUN_U4; ++i) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(buf, voff + 1024 * i, soff, 0);
    r[i] = uint4{v[0], v[1], v[2], v[3]};
  }
}

template <typename C>
__device__ __forceinline__ void as_frags(const uint4 (&kr)[C::RUN_U4], const uint4 (&vr)[C::RUN_U4],
                                         typename Mma<typename C::T>::frag (&kf)[C::KSTEPS],
                                         typename Mma<typename C::T>::frag (&vf)[2][C::PSTEPS]) {
  using Frag = typename Mma<typename C::T>::frag;
  const Frag* kp = reinterpret_cast<const Frag*>(kr);
  const Frag* vp = reinterpret_cast<const Frag*>(vr);
#pragma unroll
  for (int ks = 0; ks < C::KSTEPS; ++ks) kf[ks] = kp[ks];
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int ps = 0; ps < C::PSTEPS; ++ps) vf[db][ps] = vp[db * C::PSTEPS + ps];
}

// Softmax numerators of one 32x32 S^T block for this lane's query column. The
// queries carry the logit scale log2(e)/sqrt(64), so S holds base-2 logits t and
// p = exp2(t + nb) (SHIFT) or exp2(t) (no shift: every |t| of these queries is at
// most SHIFT_FREE_MAX, so p can neither overflow nor underflow), rounded to the
// operand type and packed as P^T fragments; l accumulates the rounded p. Keys at
// or beyond `valid` (ragged last tile) give 0.
template <typename T, bool RAGGED, bool SHIFT>
__device__ __forceinline__ void softmax_block(const f32x16& S, float nb, float& l, int key0, int valid, int lane,
                                              typename Mma<T>::frag (&pf)[32 / Mma<T>::KS]) {
  using MM = Mma<T>;
  float p[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(SHIFT ? S[r] + nb : S[r]);
  if constexpr (RAGGED) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (key0 + crow(r, lane) >= valid) p[r] = 0.f;
  }
  if constexpr (MM::KW == 1) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      pf[r] = p[r];
      l += p[r];
    }
  } else {
    const bf16x2 one2 = cvt2(1.f, 1.f);
#pragma unroll
    for (int ps = 0; ps < 2; ++ps) {
      bf16x2 pr[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        pr[v] = cvt2(p[8 * ps + 2 * v], p[8 * ps + 2 * v + 1]);
        l = __builtin_amdgcn_fdot2_f32_bf16(pr[v], one2, l, false);
      }
      const bf16x4 lo = __builtin_shufflevector(pr[0], pr[1], 0, 1, 2, 3);
      const bf16x4 hi = __builtin_shufflevector(pr[2], pr[3], 0, 1, 2, 3);
      pf[ps] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  }
}

// ---------------------------------------------------------------- token-tile staging (LDS)
// Global -> registers for tile kt. Dense: 32 rows of packed K and the packed V^T
// tile, both contiguous. Gathered: rows sel[32kt + j] of K and V (zero past nkeys;
// with per-head sets, sel and nkeys are those of the head whose columns this
// thread stages).
template <typename C, bool GATHER>
__device__ __forceinline__ void tile_load(const typename C::T* __restrict__ Kg, const typename C::T* __restrict__ Vg,
                                          const int32_t* sel, int nkeys, int M, int kt, int tid, uint4 (&rk)[C::NCK],
                                          uint4 (&rv)[C::NCK]) {
  constexpr int CPR = C::D / C::EPC;
  if constexpr (!GATHER) {
    const uint4* ks = reinterpret_cast<const uint4*>(Kg + (int64_t)kt * C::KT * C::D);
    const uint4* vs = reinterpret_cast<const uint4*>(Vg + (int64_t)kt * C::KT * C::D);
#pragma unroll
    for (int i = 0; i < C::NCK; ++i) {
      rk[i] = ks[tid + i * C::NT];
      rv[i] = vs[tid + i * C::NT];
    }
  } else {
#pragma unroll
    for (int i = 0; i < C::NCK; ++i) {
      const int c = tid + i * C::NT, j = kt * C::KT + c / CPR, e = (c % CPR) * C::EPC;
      const int64_t row = (int64_t)tok_clamp(j < nkeys ? sel[j] : 0, M) * C::D + e;
      rk[i] = j < nkeys ? *reinterpret_cast<const uint4*>(Kg + row) : uint4{0, 0, 0, 0};
      rv[i] = j < nkeys ? *reinterpret_cast<const uint4*>(Vg + row) : uint4{0, 0, 0, 0};
    }
  }
}

// Registers -> LDS buffer `buf`: K rows [KT][DPAD]; gathered 16-bit V rows [KT][VROW];
// otherwise V^T [D][VPAD] in perm_key token
// order (dense: already packed that way; gathered: each thread's 16-byte run of
// one token's V row goes to column vpos of V^T).
template <typename C, bool GATHER>
__device__ __forceinline__ void tile_store(char* lds, int buf, int tid, const int (&vpos)[C::NCK],
                                           const uint4 (&rk)[C::NCK], const uint4 (&rv)[C::NCK]) {
  using T = typename C::T;
  constexpr int CPR = C::D / C::EPC;
  constexpr int VCPR = C::KT / C::EPC;
  T* Kb = reinterpret_cast<T*>(lds + buf * C::KBYTES);
  T* Vb = reinterpret_cast<T*>(lds + 2 * C::KBYTES + buf * C::VBYTES);
#pragma unroll
  for (int i = 0; i < C::NCK; ++i) {
    const int c = tid + i * C::NT;
    *reinterpret_cast<uint4*>(Kb + (c / CPR) * C::DPAD + (c % CPR) * C::EPC) = rk[i];
    if constexpr (!GATHER) {
      *reinterpret_cast<uint4*>(Vb + (c / VCPR) * C::VPAD + (c % VCPR) * C::EPC) = rv[i];
    } else if constexpr (C::TR_V) {
      *reinterpret_cast<uint4*>(Vb + (c / CPR) * C::VROW + (c % CPR) * C::EPC) = rv[i];
    } else {
      const int e = (c % CPR) * C::EPC;
      const T* v = reinterpret_cast<const T*>(&rv[i]);
#pragma unroll
      for (int x = 0; x < C::EPC; ++x) Vb[(e + x) * C::VPAD + vpos[i]] = v[x];
    }
  }
}

// acc[r][i] += W[rows 32 r ..][..] x B[columns 32 (cb0 + i) ..]^T for NR consecutive
// row blocks of W (global memory, each through a RING-deep register prefetch ring)
// and NC column blocks of B (LDS, read BPF steps ahead, each fragment used NR times).
template <typename T, int NKS, int NR, int NC, bool PACKED, int RING = 8, int BPF = 2>
__device__ __forceinline__ void gemm_rows(const T* __restrict__ W, int ldw, const T* B, int ldb, int cb0,
                                          f32x16 (&acc)[NR][NC], int lane) {
  using MM = Mma<T>;
  using Frag = typename MM::frag;
  // A fragment of row block r, step ks. Row-major W: rows of ldw elements from the
  // block's first row; packed W: 32 x KS blocks of ldw / KS steps per row block.
  auto wfrag = [&](int r, int ks) -> Frag {
    if constexpr (PACKED)
      return *reinterpret_cast<const Frag*>(W + ((int64_t)r * (ldw / MM::KS) + ks) * (32 * MM::KS) + lane * MM::KW);
    else
      return load_frag<T>(W + (int64_t)(32 * r) * ldw + ks * MM::KS, ldw, lane);
  };
  auto bfrag = [&](int i, int ks) -> Frag { return load_frag<T>(B + (32 * (cb0 + i)) * ldb + ks * MM::KS, ldb, lane); };
  constexpr int PF = NKS < RING ? NKS : RING;        // weight steps in flight (global memory)
  constexpr int BD = NKS < BPF + 1 ? NKS : BPF + 1;  // B steps held (LDS reads BD - 1 steps ahead)
  Frag ring[NR][PF];
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int p = 0; p < PF; ++p) ring[r][p] = wfrag(r, p);
  Frag b[BD][NC];
#pragma unroll
  for (int d = 0; d < BD - 1; ++d)
#pragma unroll
    for (int i = 0; i < NC; ++i) b[d][i] = bfrag(i, d);
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    Frag a[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      a[r] = ring[r][ks % PF];
      if (ks + PF < NKS) ring[r][ks % PF] = wfrag(r, ks + PF);
    }
    if (ks + BD - 1 < NKS) {
#pragma unroll
      for (int i = 0; i < NC; ++i) b[(ks + BD - 1) % BD][i] = bfrag(i, ks + BD - 1);
    }
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int i = 0; i < NC; ++i) acc[r][i] = MM::mma(a[r], b[ks % BD][i], acc[r][i]);
  }
}

// Weight fragment of row block r, MFMA step ks, as gemm_rows reads it.
template <typename T, bool PACKED>
__device__ __forceinline__ typename Mma<T>::frag wfrag_at(const T* __restrict__ W, int ldw, int r, int ks, int lane) {
  using MM = Mma<T>;
  if constexpr (PACKED)
    return *reinterpret_cast<const typename MM::frag*>(W + ((int64_t)r * (ldw / MM::KS) + ks) * (32 * MM::KS) +
                                                       lane * MM::KW);
  else
    return load_frag<T>(W + (int64_t)(32 * r) * ldw + ks * MM::KS, ldw, lane);
}

// The first PF weight steps of W for NR row blocks, into a prefetch ring.
template <typename T, int NR, int PF, bool PACKED>
__device__ __forceinline__ void wring_fill(const T* __restrict__ W, int ldw, typename Mma<T>::frag (&ring)[NR][PF],
                                           int lane) {
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int p = 0; p < PF; ++p) ring[r][p] = wfrag_at<T, PACKED>(W, ldw, r, p, lane);
}

// gemm_rows with the weight ring passed in already holding W's first PF steps.
// With NEXT, the steps freed at the end take the first PF steps of Wn, so the
// next product of the chain starts with its weights in flight or landed: the
// loads cross the barrier between the two products (weights do not depend on
// it), instead of each product waiting for a full L2 round trip at its start.
template <typename T, int NKS, int NR, int NC, bool PACKED, int PF, bool NEXT, int BPF = 2>
__device__ __forceinline__ void gemm_rows_chained(const T* __restrict__ W, int ldw, const T* __restrict__ Wn, int ldwn,
                                                  const T* B, int ldb, int cb0, f32x16 (&acc)[NR][NC],
                                                  typename Mma<T>::frag (&ring)[NR][PF], int lane) {
  using MM = Mma<T>;
  using Frag = typename MM::frag;
  static_assert(NKS % PF == 0, "the next product's steps land in the slots its loop reads");
  auto bfrag = [&](int i, int ks) -> Frag { return load_frag<T>(B + (32 * (cb0 + i)) * ldb + ks * MM::KS, ldb, lane); };
  constexpr int BD = NKS < BPF + 1 ? NKS : BPF + 1;  // B steps held (LDS reads BD - 1 steps ahead)
  Frag b[BD][NC];
#pragma unroll
  for (int d = 0; d < BD - 1; ++d)
#pragma unroll
    for (int i = 0; i < NC; ++i) b[d][i] = bfrag(i, d);
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    Frag a[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      a[r] = ring[r][ks % PF];
      if (ks + PF < NKS)
        ring[r][ks % PF] = wfrag_at<T, PACKED>(W, ldw, r, ks + PF, lane);
      else if constexpr (NEXT)
        ring[r][ks % PF] = wfrag_at<T, PACKED>(Wn, ldwn, r, ks + PF - NKS, lane);
    }
    if (ks + BD - 1 < NKS) {
#pragma unroll
      for (int i = 0; i < NC; ++i) b[(ks + BD - 1) % BD][i] = bfrag(i, ks + BD - 1);
    }
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int i = 0; i < NC; ++i) acc[r][i] = MM::mma(a[r], b[ks % BD][i], acc[r][i]);
  }
}

// Start of row block rb, k-step ks of an epilogue weight with rows of `cols`
// elements, in the form gemm_rows<..., PACKED> reads.
template <typename C>
__device__ __forceinline__ const typename C::T* wblock(const typename C::T* W, int rb, int ks, int cols) {
  constexpr int KS = Mma<typename C::T>::KS;
  if constexpr (C::PACKED_W)
    return W + ((int64_t)rb * (cols / KS) + ks) * (32 * KS);
  else
    return W + (int64_t)(32 * rb) * cols + ks * KS;
}

// One 32-token tile for all of this wave's query blocks: S^T of the next query
// block is issued before the softmax of the current one, so MFMA and VALU work
// overlap. kf: K_h fragments (A operand), vf: V_h^T fragments.
template <typename C, bool RAGGED, bool SHIFT>
__device__ __forceinline__ void tile_compute(const typename Mma<typename C::T>::frag (&kf)[C::KSTEPS],
                                             const typename Mma<typename C::T>::frag (&vf)[2][C::PSTEPS],
                                             const typename Mma<typename C::T>::frag (&qf)[C::QB][C::KSTEPS],
                                             const float (&nb)[C::QB], f32x16 (&O)[2][C::QB], float (&l)[C::QB],
                                             int kt, int nkeys, int lane) {
  using T = typename C::T;
  using MM = Mma<T>;
  using Frag = typename MM::frag;
  const f32x16 Z = {};  // constant zero accumulator (an inline operand of the first MFMA)
  f32x16 S_next = MM::mma(kf[0], qf[0][0], Z);
#pragma unroll
  for (int ks = 1; ks < C::KSTEPS; ++ks) S_next = MM::mma(kf[ks], qf[0][ks], S_next);
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    const f32x16 S = S_next;
    if (qb + 1 < C::QB) {
      const int nq = qb + 1 < C::QB ? qb + 1 : qb;
      S_next = MM::mma(kf[0], qf[nq][0], Z);
#pragma unroll
      for (int ks = 1; ks < C::KSTEPS; ++ks) S_next = MM::mma(kf[ks], qf[nq][ks], S_next);
    }
    Frag pf[C::PSTEPS];
    softmax_block<T, RAGGED, SHIFT>(S, nb[qb], l[qb], kt * C::KT, nkeys, lane, pf);
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int ps = 0; ps < C::PSTEPS; ++ps) O[db][qb] = MM::mma(vf[db][ps], pf[ps], O[db][qb]);
  }
  if constexpr (!RAGGED && C::SCHED_ATT) {
    // Issue order for the scheduler: S of block 0; then one MFMA (S of the next
    // block, or P.V of the previous one) per slice of the softmax VALU work, so the
    // wave keeps the matrix pipe fed while it computes exponentials; P.V of the
    // last block at the end.
    constexpr int NM = (2 * C::QB - 2) * C::KSTEPS;  // MFMAs that have softmax work beside them
    constexpr int VPM = (C::QB * (SHIFT ? 48 : 32) + NM - 1) / NM;  // VALU instructions per such MFMA
    // the next tile's operand loads first, so they have the whole tile to land
    __builtin_amdgcn_sched_group_barrier(0x020, 2 * C::RUN_U4, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, C::KSTEPS, 0);
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * C::PSTEPS, 0);
  }
}

// ---------------------------------------------------------------- pipelined dense token loop
// Iteration k of the loop over 32-token tiles issues three independent pieces of
// work so that the matrix pipe and the VALU run side by side:
//   O += V(k-1) P(k-1)          P.V of the previous tile            (MFMA)
//   P(k) = exp2(S(k) [- b])      softmax numerators of this tile     (VALU)
//   S(k+1) = K(k+1) Q^T          logits of the next tile             (MFMA)
// and the loads of K(k+2) and V(k). Before the first tile P(-1) = 0 and V(-1) = 0.

template <typename C>
__device__ __forceinline__ f32x16 s_block(const typename Mma<typename C::T>::frag (&kf)[C::KSTEPS],
                                          const typename Mma<typename C::T>::frag (&q)[C::KSTEPS]) {
  using MM = Mma<typename C::T>;
  const f32x16 Z = {};
  f32x16 S = MM::mma(kf[0], q[0], Z);
#pragma unroll
  for (int ks = 1; ks < C::KSTEPS; ++ks) S = MM::mma(kf[ks], q[ks], S);
  return S;
}

// LAST: the final tile (no S of a next tile, no K load; ends with its own P.V);
// RAGGED: it is partial; SHIFT: see softmax_block.
// load_k(t, regs) / load_v(t, regs) fetch this wave's operand runs of tile t;
// after_loads(kt) runs right after them (independent work to start early).
template <typename C, bool LAST, bool RAGGED, bool SHIFT, typename LK, typename LV, typename AL>
__device__ __forceinline__ void pipe_iter(const uint4 (&k_next)[C::RUN_U4], const uint4 (&v_prev)[C::RUN_U4],
                                          uint4 (&k_load)[C::RUN_U4], uint4 (&v_load)[C::RUN_U4],
                                          LK&& load_k, LV&& load_v, AL&& after_loads,
                                          int kt, int k_tile, int nkeys, int lane,
                                          const typename Mma<typename C::T>::frag (&qf)[C::QB][C::KSTEPS],
                                          const float (&nb)[C::QB], f32x16 (&S)[C::QB],
                                          typename Mma<typename C::T>::frag (&P)[C::QB][C::PSTEPS],
                                          f32x16 (&O)[2][C::QB], float (&l)[C::QB]) {
  using T = typename C::T;
  using MM = Mma<T>;
  using Frag = typename MM::frag;
  if constexpr (!LAST) load_k(k_tile, k_load);
  load_v(kt, v_load);
  after_loads(kt);
  Frag kf[C::KSTEPS], vf[2][C::PSTEPS];
  as_frags<C>(k_next, v_prev, kf, vf);
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb)
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int ps = 0; ps < C::PSTEPS; ++ps) O[db][qb] = MM::mma(vf[db][ps], P[qb][ps], O[db][qb]);
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    Frag pn[C::PSTEPS];
    softmax_block<T, RAGGED, SHIFT>(S[qb], nb[qb], l[qb], kt * C::KT, nkeys, lane, pn);
    if constexpr (!LAST) S[qb] = s_block<C>(kf, qf[qb]);
#pragma unroll
    for (int ps = 0; ps < C::PSTEPS; ++ps) P[qb][ps] = pn[ps];
  }
  if constexpr (C::SCHED_ATT) {
    // loads first; P.V of the previous tile beside the first softmax; S of the
    // next tile beside the later ones
    constexpr int NPV = 2 * C::PSTEPS * C::QB;
    constexpr int NS = LAST ? 0 : C::KSTEPS * C::QB;
    constexpr int NM = NPV + NS;
    constexpr int VPM = (C::QB * (SHIFT ? 48 : 32) + NM - 1) / NM;
    __builtin_amdgcn_sched_group_barrier(0x020, (LAST ? 1 : 2) * C::RUN_U4, 0);
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);
    }
  }
  if constexpr (LAST) {
    Frag kf_unused[C::KSTEPS], vf_last[2][C::PSTEPS];
    as_frags<C>(k_next, v_load, kf_unused, vf_last);
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb)
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int ps = 0; ps < C::PSTEPS; ++ps) O[db][qb] = MM::mma(vf_last[db][ps], P[qb][ps], O[db][qb]);
  }
}

// Softmax shift. When B <= 64 bounds every base-2 logit of every query of a wave
// (B from Cauchy-Schwarz), p = exp2(t) lies in [2^-64, 2^64] and the wave skips
// the shift. Otherwise p = exp2(t + nb) with nb = SHIFT_FREE_MAX - t_max, t_max
// the query's largest logit (max_logits): p <= 2^64 with equality at the maximum,
// so no overflow, no vanishing row sum, and sums of up to 2^31 products p v stay
// far inside the fp32 range.
constexpr float SHIFT_FREE_MAX = 64.f;

template <int N>
__device__ __forceinline__ bool any_below(const float (&x)[N], float lim) {
  bool r = false;
#pragma unroll
  for (int i = 0; i < N; ++i) r = r || x[i] < lim;
  return r;
}

// m[qb] = max(m[qb], logits of the valid keys (index < nkeys) of one S^T block).
template <typename C>
__device__ __forceinline__ void block_max(const f32x16 (&S)[C::QB], int key0, int nkeys, int lane,
                                          float (&m)[C::QB]) {
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (key0 + crow(r, lane) < nkeys) m[qb] = fmaxf(m[qb], S[qb][r]);
}

// nb[qb] = SHIFT_FREE_MAX - (largest logit of this lane's query over the tokens),
// from the S^T products of every tile (the values the attention pass recomputes
// bit for bit). kfrags(t, kf) fetches this wave's K_h fragments of tile t; the
// next tile's are fetched while the current one is multiplied.
template <typename C, typename KF>
__device__ __forceinline__ void max_logits(KF&& kfrags, int nkeys, int lane,
                                           const typename Mma<typename C::T>::frag (&qf)[C::QB][C::KSTEPS],
                                           float (&nb)[C::QB]) {
  using Frag = typename Mma<typename C::T>::frag;
  const int nkt = (nkeys + C::KT - 1) / C::KT;
  float m[C::QB];
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) m[qb] = -__builtin_inff();
  Frag kf[C::KSTEPS], kn[C::KSTEPS];
  kfrags(0, kf);
  for (int kt = 0; kt < nkt; ++kt) {
    kfrags(kt + 1 < nkt ? kt + 1 : kt, kn);
    f32x16 S[C::QB];
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) S[qb] = s_block<C>(kf, qf[qb]);
    block_max<C>(S, kt * C::KT, nkeys, lane, m);
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) kf[ks] = kn[ks];
  }
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) nb[qb] = SHIFT_FREE_MAX - fmaxf(m[qb], __shfl_xor(m[qb], 32));
}

// This wave's K_h fragments of packed tile t (dense mode).
template <typename C>
__device__ __forceinline__ void packed_kfrags(__amdgpu_buffer_rsrc_t Kg, int t, int hw, int lane,
                                              typename Mma<typename C::T>::frag (&kf)[C::KSTEPS]) {
  using Frag = typename Mma<typename C::T>::frag;
  uint4 r[C::RUN_U4];
  load_run<C>(Kg, t, hw, lane, r);
  const Frag* kp = reinterpret_cast<const Frag*>(r);
#pragma unroll
  for (int ks = 0; ks < C::KSTEPS; ++ks) kf[ks] = kp[ks];
}

// This wave's K_h fragments of tile t of a selected token set, read straight from
// K [M][D]: lane l takes row sel[32t + l % 32] (the last token past the set's
// end; those keys are masked by block_max).
template <typename C>
__device__ __forceinline__ void gathered_kfrags(const typename C::T* __restrict__ Kg, const int32_t* sel, int nkeys,
                                                int M, int t, int hw, int lane,
                                                typename Mma<typename C::T>::frag (&kf)[C::KSTEPS]) {
  using MM = Mma<typename C::T>;
  const int row = tok_clamp(sel[min(t * C::KT + (lane & 31), nkeys - 1)], M);
  const typename C::T* p = Kg + (int64_t)row * C::D + 64 * hw + MM::KW * (lane >> 5);
#pragma unroll
  for (int ks = 0; ks < C::KSTEPS; ++ks)
    kf[ks] = *reinterpret_cast<const typename MM::frag*>(p + ks * MM::KS);
}

// Dense attention of this wave's QB query blocks over nkeys tokens starting at
// token tile kt0 (all M tokens, or one range of a split tile): the
// software-pipelined loop over 32-token tiles (see pipe_iter).
template <typename C, bool SHIFT>
__device__ __forceinline__ void dense_attention(const DecodeArgs& A, int shape, int kt0, int nkeys, int hw, int lane,
                                                const typename Mma<typename C::T>::frag (&qf)[C::QB][C::KSTEPS],
                                                const float (&nb)[C::QB], f32x16 (&O)[2][C::QB],
                                                float (&l_run)[C::QB]) {
  using Frag = typename Mma<typename C::T>::frag;
  const int nkt = (nkeys + C::KT - 1) / C::KT;
  if (nkt == 0) return;  // (no tokens: only reachable with M = 0, which the API rejects)
  // Iteration k reads K(k+1) from kb[(k+1)&1] and V(k-1) from vb[(k+1)&1] and
  // loads K(k+2) into kb[k&1], V(k) into vb[k&1]; the loop runs the full
  // iterations two at a time so buffers are static.
  const int64_t packed_bytes = (int64_t)nkt * C::KT * C::D * C::SZ;
  const int64_t first = shape * A.kv_stride + (int64_t)kt0 * C::KT * C::D * C::SZ;
  const __amdgpu_buffer_rsrc_t Kg = buffer_of((const char*)A.Kp + first, packed_bytes);
  const __amdgpu_buffer_rsrc_t Vg = buffer_of((const char*)A.Vt + first, packed_bytes);
  auto load_k = [&](int t, uint4 (&r)[C::RUN_U4]) { load_run<C>(Kg, t, hw, lane, r); };
  auto load_v = [&](int t, uint4 (&r)[C::RUN_U4]) { load_run<C>(Vg, t, hw, lane, r); };
  auto nothing = [](int) {};
  uint4 kb[2][C::RUN_U4], vb[2][C::RUN_U4];
  f32x16 S[C::QB];
  Frag P[C::QB][C::PSTEPS];
#pragma unroll
  for (int i = 0; i < C::RUN_U4; ++i) vb[1][i] = uint4{0, 0, 0, 0};
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb)
#pragma unroll
    for (int ps = 0; ps < C::PSTEPS; ++ps) P[qb][ps] = Frag{};
  load_run<C>(Kg, 0, hw, lane, kb[0]);
  load_run<C>(Kg, nkt > 1 ? 1 : 0, hw, lane, kb[1]);
  {
    Frag kf[C::KSTEPS], vf_unused[2][C::PSTEPS];
    as_frags<C>(kb[0], vb[1], kf, vf_unused);
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) S[qb] = s_block<C>(kf, qf[qb]);
  }
  int kt = 0;
  for (; kt + 2 < nkt; kt += 2) {
    pipe_iter<C, false, false, SHIFT>(kb[1], vb[1], kb[0], vb[0], load_k, load_v, nothing, kt, kt + 2, nkeys, lane, qf, nb, S, P,
                                      O, l_run);
    const int k3 = kt + 3 < nkt ? kt + 3 : nkt - 1;
    pipe_iter<C, false, false, SHIFT>(kb[0], vb[0], kb[1], vb[1], load_k, load_v, nothing, kt + 1, k3, nkeys, lane, qf, nb, S, P,
                                      O, l_run);
  }
  if (kt + 1 < nkt) {  // one more full iteration (kt even)
    pipe_iter<C, false, false, SHIFT>(kb[1], vb[1], kb[0], vb[0], load_k, load_v, nothing, kt, nkt - 1, nkeys, lane, qf, nb, S, P,
                                      O, l_run);
    ++kt;
  }
  // the last tile: softmax (masked, in case it is partial) beside P.V of the
  // previous one, then its own P.V. Its K was consumed by the previous step;
  // V of the previous tile sits in vb[(kt+1)&1] and moves to vb[1] when kt
  // is odd, so that a single instance of the step is emitted.
  if (kt & 1) {
#pragma unroll
    for (int i = 0; i < C::RUN_U4; ++i) vb[1][i] = vb[0][i];
  }
  pipe_iter<C, true, true, SHIFT>(kb[0], vb[1], kb[0], vb[0], load_k, load_v, nothing, kt, 0, nkeys, lane, qf, nb, S, P, O,
                                  l_run);
}

// dense_attention with the tile's work in two phases (16-bit types, two query
// groups): per 32-token tile k the wave runs the softmax of S(k), then the MFMAs
// S(k+1) = K(k+1) Q and O += V(k) P(k) (the same products, summed in the same
// order as dense_attention). The two waves that share a SIMD (same head, query
// groups 0 and 1) are given different instruction schedules: group 0 has a
// scheduling barrier between its softmax and its MFMAs, so the compiler overlaps
// a tile's P.V with the next tile's softmax; group 1 has one at each tile
// boundary, so it overlaps the next tile's S MFMAs with the current softmax.
// Side by side the two mixes keep the matrix pipe busier: 4-5 % less time per
// dense launch than the interleaved schedule of dense_attention, while either
// schedule on every wave was no faster (nor were hardware barriers that forced
// the waves into opposite phases: 9 % slower).
template <typename C, bool SHIFT>
__device__ __forceinline__ void dense_attention_2phase(const DecodeArgs& A, int shape, int kt0, int nkeys, int hw,
                                                       int qg, int lane,
                                                       const typename Mma<typename C::T>::frag (&qf)[C::QB][C::KSTEPS],
                                                       const float (&nb)[C::QB], f32x16 (&O)[2][C::QB],
                                                       float (&l_run)[C::QB]) {
  using T = typename C::T;
  using MM = Mma<T>;
  using Frag = typename MM::frag;
  const int nkt = (nkeys + C::KT - 1) / C::KT;
  if (nkt == 0) return;
  const int64_t packed_bytes = (int64_t)nkt * C::KT * C::D * C::SZ;
  const int64_t first = shape * A.kv_stride + (int64_t)kt0 * C::KT * C::D * C::SZ;
  const __amdgpu_buffer_rsrc_t Kg = buffer_of((const char*)A.Kp + first, packed_bytes);
  const __amdgpu_buffer_rsrc_t Vg = buffer_of((const char*)A.Vt + first, packed_bytes);
  const bool g0 = qg == 0;  // (wave-uniform)
  auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
  uint4 kb[2][C::RUN_U4], vb[2][C::RUN_U4];
  f32x16 S[C::QB];
  Frag P[C::QB][C::PSTEPS];
  load_run<C>(Kg, 0, hw, lane, kb[0]);
  load_run<C>(Vg, 0, hw, lane, vb[0]);
  load_run<C>(Kg, nkt > 1 ? 1 : 0, hw, lane, kb[1]);
  {
    const Frag* kp = reinterpret_cast<const Frag*>(kb[0]);
    Frag kf[C::KSTEPS];
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) kf[ks] = kp[ks];
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) S[qb] = s_block<C>(kf, qf[qb]);
  }
  if (!g0) fence();
  // tile kt: S holds S(kt), kn K(kt+1), vc V(kt); kl and vl receive K(kt+2), V(kt+1)
  auto tile = [&](auto last_tag, const uint4 (&kn)[C::RUN_U4], const uint4 (&vc)[C::RUN_U4],
                  uint4 (&kl)[C::RUN_U4], uint4 (&vl)[C::RUN_U4], int kt) {
    constexpr bool LAST = decltype(last_tag)::value;  // (the last tile may be partial)
    if constexpr (!LAST) {
      load_run<C>(Kg, kt + 2 < nkt ? kt + 2 : nkt - 1, hw, lane, kl);
      load_run<C>(Vg, kt + 1, hw, lane, vl);
    }
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb)
      softmax_block<T, LAST, SHIFT>(S[qb], nb[qb], l_run[qb], kt * C::KT, nkeys, lane, P[qb]);
    if (g0) fence();
    Frag kf[C::KSTEPS], vf[2][C::PSTEPS];
    as_frags<C>(kn, vc, kf, vf);
    if constexpr (!LAST) {
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb) S[qb] = s_block<C>(kf, qf[qb]);
    }
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb)
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int ps = 0; ps < C::PSTEPS; ++ps) O[db][qb] = MM::mma(vf[db][ps], P[qb][ps], O[db][qb]);
    if (!g0 && !LAST) fence();
  };
  using No = std::integral_constant<bool, false>;
  using Yes = std::integral_constant<bool, true>;
  int kt = 0;
  for (; kt + 2 < nkt; kt += 2) {  // two tiles per step, so the buffers are static
    tile(No(), kb[1], vb[0], kb[0], vb[1], kt);
    tile(No(), kb[0], vb[1], kb[1], vb[0], kt + 1);
  }
  if (kt + 1 < nkt) {  // one more full tile (kt even)
    tile(No(), kb[1], vb[0], kb[0], vb[1], kt);
    ++kt;
  }
  // the last tile, kt = nkt - 1: V(kt) is in vb[kt & 1]
  if (kt & 1) {
#pragma unroll
    for (int i = 0; i < C::RUN_U4; ++i) vb[0][i] = vb[1][i];
  }
  tile(Yes(), kb[0], vb[0], kb[1], vb[1], kt);
}

// V^T fragment (A operand of O^T += V^T P^T) for dims d0 .. d0+31 and MFMA step
// ps, read from row-major V [KT][VROW] in LDS with two transposing reads. Within
// each 16-lane group, ds_read_b64_tr_b16 gives lane i element i%4 of the 8-byte
// blocks of lanes i/4 + 4j (j = 0..3). Source lane s of group g points at row
// t0 + s/4, columns d0 + 16(g%2) + 4(s%4) .. +3, so lane i of the group receives
// V[t0 + j][d0 + 16(g%2) + i], j = 0..3: rows are dims, keys run along k. With
// t0 = 16 ps + 4(g/2) (+8 for the second read) the k slots of lane l hold keys
// 16 ps + 8(v/4) + 4(l/32) + v%4, the order in which the C layout of S^T hands
// P^T to the B operand.
template <typename C>
__device__ __forceinline__ typename Mma<typename C::T>::frag vt_frag_tr(const typename C::T* Vb, int d0, int ps,
                                                                        int lane) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  const int g = lane >> 4, s = lane & 15;
  const int t0 = 16 * ps + 4 * (g >> 1) + (s >> 2);
  const typename C::T* p = Vb + t0 * C::VROW + d0 + 16 * (g & 1) + 4 * (s & 3);
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p + 8 * C::VROW));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return *reinterpret_cast<const typename Mma<typename C::T>::frag*>(&ab);
}

// Selected-token rows of a 32-token tile t for this thread's staging chunks: the
// thread moves NCK 16-byte chunks per tile, chunk c = tid + i*NT holding elements
// (c % CPR)*EPC .. +EPC-1 of row j = 32t + c / CPR; entry i is the token index of
// that row (as stored: gather_rows clamps it to [0, M) when it is used, so that
// nothing waits for these loads before then). Rows past the set repeat its last
// token (finite values that the softmax of the last tile masks), so that no load
// is conditional: a branch around a load would end the scheduling region and wait
// for every load in flight. nkeys >= 1.
template <typename C>
__device__ __forceinline__ void tile_rows(const int32_t* sel, int nkeys, int t, int tid, int (&s)[C::NCK]) {
  constexpr int CPR = C::D / C::EPC;
#pragma unroll
  for (int i = 0; i < C::NCK; ++i) {
    const int j = t * C::KT + (tid + i * C::NT) / CPR;
    s[i] = sel[min(j, nkeys - 1)];
  }
}

// This thread's chunks of the rows s (tile_rows) of K or V ([M][D] behind the
// buffer X), into registers ...
template <typename C>
__device__ __forceinline__ void gather_rows(__amdgpu_buffer_rsrc_t X, const int (&s)[C::NCK], int M, int tid,
                                            uint4 (&r)[C::NCK]) {
  constexpr int CPR = C::D / C::EPC;
#pragma unroll
  for (int i = 0; i < C::NCK; ++i) {
    const int e = ((tid + i * C::NT) % CPR) * C::EPC;
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(X, (tok_clamp(s[i], M) * C::D + e) * C::SZ, 0, 0);
    r[i] = uint4{v[0], v[1], v[2], v[3]};
  }
}

// ... and from registers into a row-major LDS tile with rows of `ld` elements.
template <typename C>
__device__ __forceinline__ void put_rows(typename C::T* dst, int ld, int tid, const uint4 (&r)[C::NCK]) {
  constexpr int CPR = C::D / C::EPC;
#pragma unroll
  for (int i = 0; i < C::NCK; ++i) {
    const int c = tid + i * C::NT;
    *reinterpret_cast<uint4*>(dst + (c / CPR) * ld + (c % CPR) * C::EPC) = r[i];
  }
}

// Gathered attention for 16-bit types, software-pipelined. Iteration k computes
// O += V(k-1) P(k-1), P(k) = softmax(S(k)) and S(k+1) = K(k+1) Q, reading this
// wave's V(k-1) and K(k+1) operands from LDS at its start. The workgroup stages
// the selected rows through two K tiles and three V tiles in LDS: during
// iteration k every thread gathers its chunks of K tile k+2 and V tile k+1 from
// global memory (the token indices of the next K tile are fetched one iteration
// ahead), writes them into LDS at the end and the iteration closes with one
// barrier. Stage hazards: K tile k+2 replaces tile k, read in iteration k-1; V
// tile k+1 replaces tile k-2, read in iteration k-1 (iteration k reads V tile k-1,
// hence three V stages). Rows past the set repeat its last token and are masked
// in the last softmax.
template <typename C, bool SHIFT>
__device__ __forceinline__ void gathered_attention_pipe(
    const typename C::T* __restrict__ Kg, const typename C::T* __restrict__ Vg, const int32_t* sel, int nkeys, int M,
    int tid, int lane, int hw, char* lds, bool active,
    const typename Mma<typename C::T>::frag (&qf)[C::QB][C::KSTEPS], const float (&nb)[C::QB],
    f32x16 (&O)[2][C::QB], float (&l_run)[C::QB]) {
  using T = typename C::T;
  using MM = Mma<T>;
  using Frag = typename MM::frag;
  static_assert(C::TR_V && C::RUN_U4 == C::KSTEPS && C::RUN_U4 == 2 * C::PSTEPS, "one uint4 per fragment");
  const int nkt = (nkeys + C::KT - 1) / C::KT;
  if (nkt == 0) return;  // (an empty set: the API never forms work items for it)
  const __amdgpu_buffer_rsrc_t Kb = buffer_of(Kg, (int64_t)M * C::D * C::SZ);
  const __amdgpu_buffer_rsrc_t Vb = buffer_of(Vg, (int64_t)M * C::D * C::SZ);
  T* Ks = reinterpret_cast<T*>(lds);                  // two K tiles [KT][DPAD]
  T* Vs = reinterpret_cast<T*>(lds + 2 * C::KBYTES);  // three V tiles [KT][VROW]
  auto kstage = [&](int t) { return Ks + (t & 1) * (C::KBYTES / C::SZ); };
  auto vstage = [&](int t) { return Vs + ((t + 3) % 3) * (C::VBYTES / C::SZ); };  // t >= -1
  auto read_k = [&](int t, Frag (&kf)[C::KSTEPS]) {
    const T* src = kstage(t) + 64 * hw;
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) kf[ks] = load_frag<T>(src + ks * MM::KS, C::DPAD, lane);
  };
  auto read_v = [&](int t, Frag (&vf)[2][C::PSTEPS]) {
    const T* src = vstage(t);
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int ps = 0; ps < C::PSTEPS; ++ps) vf[db][ps] = vt_frag_tr<C>(src, 64 * hw + 32 * db, ps, lane);
  };
  auto pv = [&](const Frag (&vf)[2][C::PSTEPS], const Frag (&P)[C::QB][C::PSTEPS]) {
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb)
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int ps = 0; ps < C::PSTEPS; ++ps) O[db][qb] = MM::mma(vf[db][ps], P[qb][ps], O[db][qb]);
  };

  // prologue: S(0) from K tile 0 read straight from global memory (this wave's
  // head); K tile 1 and V tile 0 staged; V stage "-1" zeroed (P(-1) = 0 must not
  // meet stale bits that could be NaN)
  int sa[C::NCK], sb[C::NCK];  // token rows of V tile k+1 and K tile k+2 in iteration k
  uint4 gk[C::NCK], gv[C::NCK];
  tile_rows<C>(sel, nkeys, 0, tid, sa);
  tile_rows<C>(sel, nkeys, 1, tid, sb);
  gather_rows<C>(Vb, sa, M, tid, gv);
  gather_rows<C>(Kb, sb, M, tid, gk);
  f32x16 S[C::QB];
  if (active) {
    Frag kf[C::KSTEPS];
    const int row = tok_clamp(sel[min(lane & 31, nkeys - 1)], M);
    const int off = (row * C::D + 64 * hw + MM::KW * (lane >> 5)) * C::SZ;
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(Kb, off + ks * MM::KS * C::SZ, 0, 0);
      const uint4 u{v[0], v[1], v[2], v[3]};
      kf[ks] = *reinterpret_cast<const Frag*>(&u);
    }
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) S[qb] = s_block<C>(kf, qf[qb]);
  }
  {
    uint4 z[C::NCK];
#pragma unroll
    for (int i = 0; i < C::NCK; ++i) z[i] = uint4{0, 0, 0, 0};
    put_rows<C>(vstage(-1), C::VROW, tid, z);
  }
  put_rows<C>(vstage(0), C::VROW, tid, gv);
  put_rows<C>(kstage(1), C::DPAD, tid, gk);
#pragma unroll
  for (int i = 0; i < C::NCK; ++i) sa[i] = sb[i];
  tile_rows<C>(sel, nkeys, 2, tid, sb);
  __syncthreads();

  // staging of one loop iteration k (every wave takes part)
  auto stage_next = [&](int k, auto work) {
    int sn[C::NCK];
    gather_rows<C>(Vb, sa, M, tid, gv);
    gather_rows<C>(Kb, sb, M, tid, gk);
    tile_rows<C>(sel, nkeys, k + 3, tid, sn);
    work();
    put_rows<C>(kstage(k + 2), C::DPAD, tid, gk);
    put_rows<C>(vstage(k + 1), C::VROW, tid, gv);
#pragma unroll
    for (int i = 0; i < C::NCK; ++i) {
      sa[i] = sb[i];
      sb[i] = sn[i];
    }
    __syncthreads();
  };
  if (!active) {
    // (no queries in this wave: it only keeps the workgroup's staging and barriers)
    for (int k = 0; k + 1 < nkt; ++k) stage_next(k, [] {});
    __syncthreads();
    return;
  }
  Frag P[C::QB][C::PSTEPS];
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb)
#pragma unroll
    for (int ps = 0; ps < C::PSTEPS; ++ps) P[qb][ps] = Frag{};
  for (int k = 0; k + 1 < nkt; ++k) {
    Frag vf[2][C::PSTEPS], kf[C::KSTEPS];
    read_v(k - 1, vf);
    read_k(k + 1, kf);
    stage_next(k, [&] {
      pv(vf, P);
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb) {
        softmax_block<T, false, SHIFT>(S[qb], nb[qb], l_run[qb], k * C::KT, nkeys, lane, P[qb]);
        S[qb] = s_block<C>(kf, qf[qb]);
      }
      if constexpr (C::SCHED_ATT) {
        // operand reads and gathers first, then P.V of the previous tile beside the
        // first softmax and S of the next tile beside the later ones
        constexpr int NM = (2 * C::PSTEPS + C::KSTEPS) * C::QB;
        constexpr int VPM = (C::QB * (SHIFT ? 48 : 32) + NM - 1) / NM;
        __builtin_amdgcn_sched_group_barrier(0x100, 4 * C::PSTEPS + C::KSTEPS, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 3 * C::NCK, 0);
#pragma unroll
        for (int i = 0; i < NM; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);
        }
      }
    });
  }
  {
    // last tile (ragged): P.V of the one before, its softmax and its own P.V
    const int k = nkt - 1;
    Frag vf[2][C::PSTEPS];
    read_v(k - 1, vf);
    pv(vf, P);
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb)
      softmax_block<T, true, SHIFT>(S[qb], nb[qb], l_run[qb], k * C::KT, nkeys, lane, P[qb]);
    read_v(k, vf);
    pv(vf, P);
  }
  __syncthreads();
}

// Attention over one block's selected token set: 32-token tiles gathered into
// an LDS double buffer (V transposed on the way in), one barrier per tile.
// sel_st / nk_st: the token set this thread stages (its head's with per-head
// sets); nkeys: this wave's count (its softmax masks keys past it); nkt: tiles
// of the largest set of the workgroup (every wave runs them for the barriers).
template <typename C, bool SHIFT>
__device__ __forceinline__ void gathered_attention(const typename C::T* __restrict__ Kg,
                                                   const typename C::T* __restrict__ Vg, const int32_t* sel_st,
                                                   int nk_st, int nkeys, int nkt, int M, int tid, int lane, int hw,
                                                   char* lds, const int (&vpos)[C::NCK], bool active,
                                                   const typename Mma<typename C::T>::frag (&qf)[C::QB][C::KSTEPS],
                                                   const float (&nb)[C::QB], f32x16 (&O)[2][C::QB],
                                                   float (&l_run)[C::QB]) {
  using T = typename C::T;
  using MM = Mma<T>;
  using Frag = typename MM::frag;
  uint4 rk[C::NCK], rv[C::NCK];
  tile_load<C, true>(Kg, Vg, sel_st, nk_st, M, 0, tid, rk, rv);
  tile_store<C, true>(lds, 0, tid, vpos, rk, rv);
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    // prefetch the next tile (clamped: the last step reloads its own tile)
    tile_load<C, true>(Kg, Vg, sel_st, nk_st, M, kt + 1 < nkt ? kt + 1 : kt, tid, rk, rv);
    const T* Kb = reinterpret_cast<const T*>(lds + (kt & 1) * C::KBYTES);
    const T* Vb = reinterpret_cast<const T*>(lds + 2 * C::KBYTES + (kt & 1) * C::VBYTES);
    if (active) {  // (a wave whose queries are all past the item's end only stages tiles)
    Frag kf[C::KSTEPS], vf[2][C::PSTEPS];
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) kf[ks] = load_frag<T>(Kb + 64 * hw + ks * MM::KS, C::DPAD, lane);
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int ps = 0; ps < C::PSTEPS; ++ps) {
        if constexpr (C::TR_V)
          vf[db][ps] = vt_frag_tr<C>(Vb, 64 * hw + 32 * db, ps, lane);
        else
          vf[db][ps] = load_frag<T>(Vb + (64 * hw + 32 * db) * C::VPAD + ps * MM::KS, C::VPAD, lane);
      }
    if ((kt + 1) * C::KT > nkeys)
      tile_compute<C, true, SHIFT>(kf, vf, qf, nb, O, l_run, kt, nkeys, lane);
    else
      tile_compute<C, false, SHIFT>(kf, vf, qf, nb, O, l_run, kt, nkeys, lane);
    }
    // the other buffer was last read before the previous barrier
    tile_store<C, true>(lds, (kt + 1) & 1, tid, vpos, rk, rv);
    __syncthreads();
  }
}

// RAGGED: a batch whose shapes have their own device-side counts (tile_prefix);
// a separate instance, so that the single-shape kernels keep their registers.
template <typename C, bool GATHER, bool RAGGED>
__global__ __launch_bounds__(C::NT) void decode_kernel(DecodeArgs A) {
  extern __shared__ __align__(16) char lds[];
  using T = typename C::T;
  using MM = Mma<T>;
  using Frag = typename MM::frag;
  constexpr int KS = C::KSTEPS;

  const int tid0 = threadIdx.x, lane0 = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid0 >> 6);  // wave-uniform: scalar registers
  const int hw = wave % C::H, qg = wave / C::H;
  const int nbatch = A.batch > 1 ? A.batch : 1;
  const int64_t nq_all = A.d_N ? (int64_t)*A.d_N : A.N;
  const int64_t tps = (nq_all + C::BQ - 1) / C::BQ;  // dense tiles per shape (same-size batch)
  const int64_t n_tiles = RAGGED ? A.tile_prefix[nbatch]
                                 : A.items ? (A.d_n_items ? (int64_t)*A.d_n_items : A.n_tiles) : tps * nbatch;
  const T* __restrict__ Wo = (const T*)A.Wo;
  const T* __restrict__ W1 = (const T*)A.W1;
  const T* __restrict__ W2 = (const T*)A.W2;

  const float2* gtab = reinterpret_cast<const float2*>(lds + C::GTAB);
  if constexpr (C::GELU_TABLE) gelu_table_fill(reinterpret_cast<float2*>(lds + C::GTAB), tid0, C::NT);
  // (the first barrier of the tile loop orders the fill before any lookup)

  int vpos[C::NCK] = {};
  if constexpr (GATHER) {
    constexpr int CPR = C::D / C::EPC;
#pragma unroll
    for (int i = 0; i < C::NCK; ++i) vpos[i] = key_pos<T>((tid0 + i * C::NT) / CPR);
  }

  // work units: whole tiles, then (dense tail split) split_tiles tiles of `split`
  // token ranges each, a tile's ranges on consecutive units. Workgroups take units
  // in order from the counter A.queue (required in gathered mode, where work items
  // differ in set size and query count; with dense tiles it lets faster compute
  // units take more of them; without it, units go round-robin): thread 0 fetches
  // the next index at the start of each unit (the atomic's latency hides behind
  // the unit) and the loop's end hands it to the workgroup through LDS.
  const int64_t n_whole = n_tiles - A.split_tiles;
  const int64_t n_units = n_whole + A.split_tiles * A.split;
  __shared__ int64_t unit_slot;
  int64_t pending = 0;  // thread 0: the next work item (gathered)
  const bool dyn = GATHER || A.queue != nullptr;  // (uniform)
  auto fetch = [&] {
    if (dyn && tid0 == 0) pending = (int64_t)atomicAdd(A.queue, 1ull);
  };
  auto next_unit = [&](int64_t u) -> int64_t {
    if (!dyn) return u + gridDim.x;
    if (tid0 == 0) unit_slot = pending;
    __syncthreads();
    const int64_t v = unit_slot;
    __syncthreads();  // (read by every thread before thread 0 writes it again)
    return v;
  };
  int64_t first = blockIdx.x;
  if (dyn) {
    fetch();
    first = next_unit(0);
  }
  for (int64_t unit = first; unit < n_units; unit = next_unit(unit)) {
    fetch();
    int64_t tile = unit;
    int part = -1;  // this unit's token range of a split tile, or -1
    if (!GATHER && unit >= n_whole) {
      tile = n_whole + (unit - n_whole) / A.split;
      part = (int)((unit - n_whole) % A.split);
    }
    // Thread and lane indices are re-derived opaquely in each phase, so that the
    // address arithmetic of one phase is neither hoisted out of the tile loop
    // nor shared with another phase: otherwise it stays live across the token
    // loop, whose registers are all taken.
    int tid = opaque(tid0), lane = opaque(lane0);
    int64_t q0, q1;
    int row = -1, shape = 0;
    int64_t nq = nq_all;
    const Item* items = A.items;
    const int32_t* sel_cnt = A.sel_cnt;
    const int32_t* sel_idx = A.sel_idx;
    const T* __restrict__ Kg = (const T*)A.Kp;
    const T* __restrict__ Vg = (const T*)A.Vt;
    if constexpr (RAGGED) {
      // the shape whose tiles hold this one: tile_prefix[shape] <= tile <
      // tile_prefix[shape + 1] (a shape without tiles has equal neighbours and is
      // passed over); then that shape's count, items, selection and K/V
      int lo = 0;
#pragma unroll
      for (int step = 2048; step >= 1; step >>= 1) {  // (batches of at most 4096 shapes)
        const int mid = lo + step;
        lo = mid < nbatch && A.tile_prefix[mid] <= tile ? mid : lo;
      }
      shape = __builtin_amdgcn_readfirstlane(lo);
      tile -= A.tile_prefix[shape];
      nq = A.d_N[shape * A.cnt_stride];
      items = reinterpret_cast<const Item*>((const char*)A.items + shape * A.items_stride);
      sel_cnt = reinterpret_cast<const int32_t*>((const char*)A.sel_cnt + shape * A.sel_stride);
      sel_idx = reinterpret_cast<const int32_t*>((const char*)A.sel_idx + shape * A.sel_stride);
      Kg = reinterpret_cast<const T*>((const char*)A.Kp + shape * A.kv_stride);
      Vg = reinterpret_cast<const T*>((const char*)A.Vt + shape * A.kv_stride);
    }
    if (A.items) {
      // one item per workgroup: its fields are uniform (scalar registers)
      const Item it = items[tile];
      q0 = __builtin_amdgcn_readfirstlane(it.q0);
      q1 = __builtin_amdgcn_readfirstlane(it.q1);
      row = __builtin_amdgcn_readfirstlane(it.row);
      // (uniform: the whole workgroup skips a malformed item, before any barrier)
      if (!VDM_BOUND(q0 >= 0 && q0 <= q1 && q1 <= nq && q1 - q0 <= C::BQ, BC_DECODE_ITEM)) continue;
      if (!VDM_BOUND(!GATHER || row >= 0, BC_DECODE_ROW)) continue;
    } else {
      int64_t lt = tile;
      if (!RAGGED && nbatch > 1) {
        shape = (int)(tile / tps);
        lt = tile - (int64_t)shape * tps;
      }
      q0 = lt * C::BQ;
      q1 = q0 + C::BQ < nq ? q0 + C::BQ : nq;
    }
    const float kmax = A.kmax[shape * (RAGGED ? A.kmax_stride : C::H) + hw];

    // ---------------------------------------------------------------- Q = Wq e(p)
    // (scaled by log2(e)/sqrt(64) before the one rounding, so logits come out in base 2)
    auto query_src = [&] {  // (rebuilt where used: not held across the token loop)
      QuerySrc q = A.qs;
      if constexpr (RAGGED) q.list = reinterpret_cast<const int32_t*>((const char*)A.qs.list + shape * A.list_stride);
      return q;
    };
    embed_qproj<T, C::BQ, C::D, C::NT>(query_src(), q0, q1, (const T*)A.Wq, lds, tid, SOFTMAX_SCALE_LOG2);
    lane = opaque(lane);
    Frag qf[C::QB][KS];
    float nb[C::QB];  // the fixed softmax shift of this lane's query (if one is needed), per block
    {
      const T* Qs = reinterpret_cast<const T*>(lds + EmbedLds<T, C::BQ, C::D>::QS);
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb) {
        float n2 = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          qf[qb][ks] = load_frag<T>(Qs + (qg * C::QW + 32 * qb) * C::DPAD + 64 * hw + ks * MM::KS, C::DPAD, lane);
          if constexpr (MM::KW == 1) {
            n2 += qf[qb][ks] * qf[qb][ks];
          } else {
#pragma unroll
            for (int v = 0; v < MM::KW; ++v) n2 += (float)qf[qb][ks][v] * (float)qf[qb][ks][v];
          }
        }
        n2 += __shfl_xor(n2, 32);
        // B: upper bound of the base-2 logit over all tokens (Cauchy-Schwarz with
        // the head's largest key norm), inflated to cover fp32 rounding
        nb[qb] = SHIFT_FREE_MAX - 1.00390625f * sqrtf(n2) * kmax;
      }
    }
    __syncthreads();

    // ---------------------------------------------------------------- attention
    // gathered: this wave's token set (per-head sets: selection row row * H + head)
    const int64_t srow = GATHER ? (A.heads ? (int64_t)row * C::H + hw : row) : 0;
    const int nkeys = GATHER ? min(max(sel_cnt[srow], 0), A.cap) : A.M;
    if (GATHER) (void)VDM_BOUND(sel_cnt[srow] >= 0 && sel_cnt[srow] <= A.cap, BC_DECODE_SET);
    const int32_t* sel = GATHER ? sel_idx + srow * A.cap : nullptr;

    f32x16 O[2][C::QB];
    float l_run[C::QB];
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) {
      O[0][qb] = zero16();
      O[1][qb] = zero16();
      l_run[qb] = 0.f;
    }

    // logits of every query of this wave within +-SHIFT_FREE_MAX: no shift;
    // otherwise the shift comes from each query's largest logit
    const bool shift = __builtin_amdgcn_ballot_w64(any_below(nb, 0.f)) != 0;
    const bool active = qg * C::QW < q1 - q0;  // this wave has queries in the tile
    if (shift && active && nkeys > 0) {
      if constexpr (!GATHER) {
        const int64_t packed_bytes = (int64_t)((nkeys + C::KT - 1) / C::KT) * C::KT * C::D * C::SZ;
        const __amdgpu_buffer_rsrc_t Kb = buffer_of((const char*)A.Kp + shape * A.kv_stride, packed_bytes);
        max_logits<C>([&](int t, Frag(&kf)[KS]) { packed_kfrags<C>(Kb, t, hw, lane, kf); }, nkeys, lane, qf, nb);
      } else {
        max_logits<C>([&](int t, Frag(&kf)[KS]) { gathered_kfrags<C>(Kg, sel, nkeys, A.M, t, hw, lane, kf); },
                      nkeys, lane, qf, nb);
      }
    }
    if constexpr (!GATHER) {
      // a split tile's range: token tiles [kt0, kt0 + per) (the shift above came
      // from every token, so all ranges share it and their sums add plainly)
      int kt0 = 0, nk = nkeys;
      if (part >= 0) {
        const int nkt = (nkeys + C::KT - 1) / C::KT, per = (nkt + A.split - 1) / A.split;
        kt0 = min(part * per, nkt);
        nk = max(min(nkeys, (kt0 + per) * C::KT) - kt0 * C::KT, 0);
      }
      if (!active) {
        // (every query of this wave lies past the tile's end: nothing to attend)
      } else if constexpr (C::SCHED_ATT) {
        if (shift)
          dense_attention_2phase<C, true>(A, shape, kt0, nk, hw, qg, lane, qf, nb, O, l_run);
        else
          dense_attention_2phase<C, false>(A, shape, kt0, nk, hw, qg, lane, qf, nb, O, l_run);
      } else if (shift) {
        dense_attention<C, true>(A, shape, kt0, nk, hw, lane, qf, nb, O, l_run);
      } else {
        dense_attention<C, false>(A, shape, kt0, nk, hw, lane, qf, nb, O, l_run);
      }
      if (part >= 0) {
        // partial O and row sums to this range's slot; the last range to arrive
        // adds all of them in range order (the same sums whichever arrives last)
        constexpr int NCOMP = 2 * C::QB * 16 + C::QB;
        const int64_t tslot = (tile - n_whole) * A.split;
        float* mine = A.part + ((tslot + part) * C::NW + wave) * NCOMP * 64 + lane;
#pragma unroll
        for (int qb = 0; qb < C::QB; ++qb) {
#pragma unroll
          for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) mine[((qb * 2 + db) * 16 + r) * 64] = O[db][qb][r];
          mine[(2 * C::QB * 16 + qb) * 64] = l_run[qb];
        }
        __threadfence();  // release: the partials before the arrival count
        __syncthreads();
        int* flag = reinterpret_cast<int*>(lds + C::RED);
        if (tid == 0) *flag = atomicAdd(&A.part_cnt[tile - n_whole], 1) == A.split - 1;
        __syncthreads();
        const bool last = *flag != 0;
        __syncthreads();  // (the flag's word is reused by the head)
        if (!last) continue;  // (uniform) another range finishes this tile
        __threadfence();      // acquire: the other ranges' partials
#pragma unroll
        for (int qb = 0; qb < C::QB; ++qb) {
          O[0][qb] = zero16();
          O[1][qb] = zero16();
          l_run[qb] = 0.f;
        }
        for (int pr = 0; pr < A.split; ++pr) {
          const float* src = A.part + ((tslot + pr) * C::NW + wave) * NCOMP * 64 + lane;
#pragma unroll
          for (int qb = 0; qb < C::QB; ++qb) {
#pragma unroll
            for (int db = 0; db < 2; ++db)
#pragma unroll
              for (int r = 0; r < 16; ++r) O[db][qb][r] += src[((qb * 2 + db) * 16 + r) * 64];
            l_run[qb] += src[(2 * C::QB * 16 + qb) * 64];
          }
        }
      }
    } else {
      // (both variants pass the same barriers, so waves may take different ones)
      if (A.heads) {
        // per-head sets: this thread stages the columns of head hs (the same head
        // for all of its chunks), with that head's set; tiles of the largest set
        constexpr int CPR = C::D / C::EPC;
        const int hs = ((tid % CPR) * C::EPC) / 64;
        const int64_t st_row = (int64_t)row * C::H + hs;
        const int nk_st = min(max(sel_cnt[st_row], 0), A.cap);
        int nmax = 0;
#pragma unroll
        for (int h = 0; h < C::H; ++h) nmax = max(nmax, min(max(sel_cnt[(int64_t)row * C::H + h], 0), A.cap));
        const int nkt = (nmax + C::KT - 1) / C::KT;
        const int32_t* sel_st = sel_idx + st_row * A.cap;
        if (shift)
          gathered_attention<C, true>(Kg, Vg, sel_st, nk_st, nkeys, nkt, A.M, tid, lane, hw, lds, vpos, active, qf, nb,
                                      O, l_run);
        else
          gathered_attention<C, false>(Kg, Vg, sel_st, nk_st, nkeys, nkt, A.M, tid, lane, hw, lds, vpos, active, qf,
                                       nb, O, l_run);
      } else if constexpr (C::TR_V) {
        if (shift)
          gathered_attention_pipe<C, true>(Kg, Vg, sel, nkeys, A.M, tid, lane, hw, lds, active, qf, nb, O, l_run);
        else
          gathered_attention_pipe<C, false>(Kg, Vg, sel, nkeys, A.M, tid, lane, hw, lds, active, qf, nb, O, l_run);
      } else {
        const int nkt = (nkeys + C::KT - 1) / C::KT;
        if (shift)
          gathered_attention<C, true>(Kg, Vg, sel, nkeys, nkeys, nkt, A.M, tid, lane, hw, lds, vpos, active, qf, nb, O,
                                      l_run);
        else
          gathered_attention<C, false>(Kg, Vg, sel, nkeys, nkeys, nkt, A.M, tid, lane, hw, lds, vpos, active, qf, nb,
                                       O, l_run);
      }
    }

    // ---------------------------------------------------------------- o = sum p v / sum p
    tid = opaque(tid);
    lane = opaque(lane);
    // this wave's epilogue tiles: weight row blocks rb0 .. rb0 + RPW - 1, column
    // blocks cb0 .. cb0 + NCB - 1. In gathered mode, when every wave covers all
    // column blocks, a work item with at most half a tile of queries computes only
    // the first half of the column blocks.
    const int rb0 = C::TPW >= C::CB ? wave * C::RPW : (wave * C::TPW) / C::CB;
    const int cb0 = C::TPW >= C::CB ? 0 : (wave * C::TPW) % C::CB;
    const int rh0 = C::TPH >= C::CB ? wave * C::RPH : (wave * C::TPH) / C::CB;
    const int ch0 = C::TPH >= C::CB ? 0 : (wave * C::TPH) % C::CB;
    // one weight prefetch ring runs through the chain Wo, W1, W2, W1, ... W2; its
    // first Wo steps are issued before the O stores and their barrier
    constexpr int NKD = C::D / MM::KS;
    constexpr int PFE = NKD < 4 ? NKD : 4;
    static_assert(C::FC == C::D && C::RPH == C::RPW, "one ring shape serves Wo, W1 and W2");
    Frag wring[C::RPW][PFE];
    wring_fill<T, C::RPW, PFE, C::PACKED_W>(wblock<C>(Wo, rb0, 0, C::D), C::D, wring, lane);
    T* Ob = reinterpret_cast<T*>(lds + C::OBUF);
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) {
      // (an empty token set, sel_cnt = 0, has l = 0 and gives o = 0)
      const float lsum = l_run[qb] + __shfl_xor(l_run[qb], 32);
      const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        O[db][qb] *= inv;
        store_ct<T>(Ob + (qg * C::QW + 32 * qb) * C::DPAD + 64 * hw + 32 * db, C::DPAD, O[db][qb], lane);
      }
    }
    __syncthreads();

    // ---------------------------------------------------------------- a = Wo o  (kept in fp32 as y)
    T* Ab = reinterpret_cast<T*>(lds + C::ABUF);
    T* Hb = reinterpret_cast<T*>(lds + C::OBUF);
    float* red = reinterpret_cast<float*>(lds + C::RED);
    auto epilogue = [&](auto ncb_tag) {
    constexpr int NCB = decltype(ncb_tag)::value;
    constexpr int NCH = C::CPH == C::CB ? NCB : C::CPH;
    f32x16 Y[C::RPW][NCB];
#pragma unroll
    for (int r = 0; r < C::RPW; ++r)
#pragma unroll
      for (int i = 0; i < NCB; ++i) Y[r][i] = zero16();
    gemm_rows_chained<T, NKD, C::RPW, NCB, C::PACKED_W, PFE, true>(
        wblock<C>(Wo, rb0, 0, C::D), C::D, wblock<C>(W1, rh0, 0, C::D), C::D, Ob, C::DPAD, cb0, Y, wring, lane);
#pragma unroll
    for (int r = 0; r < C::RPW; ++r)
#pragma unroll
      for (int i = 0; i < NCB; ++i)
        store_ct<T>(Ab + (32 * (cb0 + i)) * C::DPAD + 32 * (rb0 + r), C::DPAD, Y[r][i], lane);
    __syncthreads();

    // ---------------------------------------------------------------- y = a + W2 GELU(W1 a)
    // (hidden chunks of FC; the last W2 product ends the weight chain)
    auto chunk = [&](int f0, auto last_tag) {
      constexpr bool LASTC = decltype(last_tag)::value;
      f32x16 Hc[C::RPH][NCH];
#pragma unroll
      for (int r = 0; r < C::RPH; ++r)
#pragma unroll
        for (int j = 0; j < NCH; ++j) Hc[r][j] = zero16();
      gemm_rows_chained<T, NKD, C::RPH, NCH, C::PACKED_W, PFE, true>(
          wblock<C>(W1, f0 / 32 + rh0, 0, C::D), C::D, wblock<C>(W2, rb0, f0 / MM::KS, A.F), A.F, Ab, C::DPAD, ch0,
          Hc, wring, lane);
#pragma unroll
      for (int r = 0; r < C::RPH; ++r)
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
          gelu_tile<C>(Hc[r][j], gtab);
          store_ct<T>(Hb + (32 * (ch0 + j)) * C::HPAD + 32 * (rh0 + r), C::HPAD, Hc[r][j], lane);
        }
      __syncthreads();
      gemm_rows_chained<T, C::FC / MM::KS, C::RPW, NCB, C::PACKED_W, PFE, !LASTC>(
          wblock<C>(W2, rb0, f0 / MM::KS, A.F), A.F, wblock<C>(W1, (f0 + C::FC) / 32 + rh0, 0, C::D), C::D, Hb,
          C::HPAD, cb0, Y, wring, lane);
      __syncthreads();
    };
    int f0 = 0;
    for (; f0 + C::FC < A.F; f0 += C::FC) chunk(f0, std::false_type());
    chunk(f0, std::true_type());  // (F >= FC, checked when the decoder is created)

    // ---------------------------------------------------------------- net = w_head . y, SDF
    {
      float s[C::CPW];
#pragma unroll
      for (int i = 0; i < C::CPW; ++i) s[i] = 0.f;
#pragma unroll
      for (int r = 0; r < C::RPW; ++r) {
        float w[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) w[k] = A.w_head[32 * (rb0 + r) + crow(k, lane)];
#pragma unroll
        for (int i = 0; i < NCB; ++i)
#pragma unroll
          for (int k = 0; k < 16; ++k) s[i] += w[k] * Y[r][i][k];
      }
#pragma unroll
      for (int i = 0; i < C::CPW; ++i) {
        s[i] += __shfl_xor(s[i], 32);
        if (lane < 32) red[wave * C::BQ + 32 * (cb0 + i) + lane] = s[i];
      }
      // column blocks this wave does not cover contribute zero
      for (int cb = 0; cb < C::CB; ++cb)
        if ((cb < cb0 || cb >= cb0 + C::CPW) && lane < 32) red[wave * C::BQ + 32 * cb + lane] = 0.f;
    }
    };
    if constexpr (C::CPW == C::CB && GATHER) {
      // (work items of a block's token set often end part-way through a tile: the
      // epilogue runs on the item's 32-query column blocks only; wave-uniform)
      const int ncb = (int)((q1 - q0 + 31) / 32);
      if constexpr (C::CB == 4) {
        if (ncb > 3)
          epilogue(std::integral_constant<int, 4>{});
        else if (ncb == 3)
          epilogue(std::integral_constant<int, 3>{});
        else if (ncb == 2)
          epilogue(std::integral_constant<int, 2>{});
        else
          epilogue(std::integral_constant<int, 1>{});
      } else if (2 * ncb > C::CB) {
        epilogue(std::integral_constant<int, C::CB>{});
      } else {
        epilogue(std::integral_constant<int, C::CB / 2>{});
      }
    } else {
      epilogue(std::integral_constant<int, C::CPW>{});
    }
    __syncthreads();
    const QuerySrc qs = query_src();
    for (int t = tid; t < C::BQ; t += C::NT) {
      const int64_t q = q0 + t;
      if (q < q1) {
        float net = 0.f;
#pragma unroll
        for (int w = 0; w < C::NW; ++w) net += red[w * C::BQ + t];
        const Coords p = query_coords(qs, q);
        const float sdf = analytic_sdf(p, A.prims) + A.net_scale * net;
        int64_t o = q;
        if (A.scatter) o = qs.mode == 1 ? q : (int64_t)qs.list[q];
        A.out[o + shape * A.out_stride] = sdf;
      }
    }
    __syncthreads();
  }
}

typedef DecCfg<bf16, 4, 8, 64, 256> CfgB256;
typedef DecCfg<bf16, 1, 4, 32, 64> CfgB64;
typedef DecCfg<float, 1, 4, 32, 64> CfgF64;

// workgroups of the persistent decode grid
template <typename C, bool GATHER, bool RAGGED = false>
static hipError_t decode_grid(int64_t* grid) {
  constexpr int lds = C::LDS;
  static bool attr = false;
  const void* fn = reinterpret_cast<const void*>(&decode_kernel<C, GATHER, RAGGED>);
  if (!attr) {
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    attr = true;
  }
  int per_cu = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_kernel<C, GATHER, RAGGED>, C::NT, lds);
  if (e != hipSuccess) return e;
  if (per_cu < 1) per_cu = 1;
  *grid = (int64_t)dev_info().cus * per_cu;
  return hipSuccess;
}

template <typename C, bool GATHER, bool RAGGED = false>
static hipError_t run(const DecodeArgs& a, hipStream_t s) {
  constexpr int lds = C::LDS;
  if (!RAGGED && a.batch > 1 && a.tile_prefix) return run<C, GATHER, true>(a, s);
  int64_t grid = 0;
  hipError_t e = decode_grid<C, GATHER, RAGGED>(&grid);
  if (e != hipSuccess) return e;
  if (!a.d_N && !a.d_n_items) {
    const int64_t host_tiles = a.items ? a.n_tiles : (a.N + C::BQ - 1) / C::BQ * (a.batch > 1 ? a.batch : 1);
    const int64_t host_units = host_tiles + a.split_tiles * (a.split - 1);
    if (host_units < grid) grid = host_units;
  }
  if (grid < 1) return hipSuccess;
  hipLaunchKernelGGL((decode_kernel<C, GATHER, RAGGED>), dim3((unsigned)grid), dim3(C::NT), lds, s, a);
  return hipGetLastError();
}

SplitPlan decode_split_plan(int dtype, int D, int64_t M, int64_t n_tiles) {
  SplitPlan p;
  if (dtype != VDM_BF16 || D != 256 || M < 8192 || n_tiles < 1) return p;
  int64_t G = 0;
  if (decode_grid<CfgB256, false>(&G) != hipSuccess || G < 2) return p;
  const int64_t tail = n_tiles % G;  // the last round's tiles (all of them when fewer than G)
  if (tail == 0 || 2 * tail > G) return p;
  const int64_t nkt = (M + CfgB256::KT - 1) / CfgB256::KT;
  int64_t parts = G / tail;
  if (parts > nkt / 16) parts = nkt / 16;  // ranges of at least 16 token tiles
  if (parts > 16) parts = 16;
  if (parts < 2) return p;
  constexpr int NCOMP = 2 * CfgB256::QB * 16 + CfgB256::QB;
  p.parts = (int)parts;
  p.tiles = tail;
  p.part_bytes = (size_t)tail * parts * CfgB256::NW * NCOMP * 64 * sizeof(float);
  p.cnt_bytes = ((size_t)tail * sizeof(int32_t) + 255) / 256 * 256;
  return p;
}

hipError_t launch_decode(int dtype, int D, bool gathered, const DecodeArgs& a, hipStream_t s) {
  if (gathered && !a.queue) return hipErrorInvalidValue;  // (the work-item counter is required)
  if (dtype == VDM_BF16 && D == 256) return gathered ? run<CfgB256, true>(a, s) : run<CfgB256, false>(a, s);
  if (dtype == VDM_BF16 && D == 64) return gathered ? run<CfgB64, true>(a, s) : run<CfgB64, false>(a, s);
  return gathered ? run<CfgF64, true>(a, s) : run<CfgF64, false>(a, s);
}

// ---------------------------------------------------------------- head of the local decoder
// y = h + W2 GELU(W1 h), net = w_head . y, SDF = analytic + net_scale net for
// fused features h [N][256] (bf16) of the local KNN decoder: the epilogue of
// decode_kernel with h in place of Wo o, one 128-query tile per workgroup
// iteration, the weights streamed once per tile.
template <typename C>
__global__ __launch_bounds__(C::NT) void local_head_kernel(HeadArgs A) {
  extern __shared__ __align__(16) char lds[];
  using T = typename C::T;
  using MM = Mma<T>;
  static_assert(C::D == 256 && C::PACKED_W && C::GELU_TABLE && C::CPW == C::CB, "the 256-wide bf16 head");
  const int tid0 = threadIdx.x, lane0 = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid0 >> 6);
  const T* __restrict__ W1 = (const T*)A.W1;
  const T* __restrict__ W2 = (const T*)A.W2;
  const T* __restrict__ Hg = (const T*)A.h;
  const float2* gtab = reinterpret_cast<const float2*>(lds + C::GTAB);
  gelu_table_fill(reinterpret_cast<float2*>(lds + C::GTAB), tid0, C::NT);
  T* Ab = reinterpret_cast<T*>(lds + C::ABUF);
  T* Hb = reinterpret_cast<T*>(lds + C::OBUF);
  float* red = reinterpret_cast<float*>(lds + C::RED);
  const int64_t n_tiles = (A.N + C::BQ - 1) / C::BQ;
  constexpr int NCB = C::CB, NCH = C::CPH;
  for (int64_t tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
    int tid = opaque(tid0), lane = opaque(lane0);
    const int64_t q0 = tile * C::BQ;
    const int64_t q1 = q0 + C::BQ < A.N ? q0 + C::BQ : A.N;
    // h rows of the tile into Ab [BQ][DPAD] (rows past the end: zero)
    constexpr int CPR = C::D * C::SZ / 16;
    for (int c = tid; c < C::BQ * CPR; c += C::NT) {
      const int r = c / CPR, e = (c % CPR) * (16 / C::SZ);
      const uint4 v = q0 + r < q1 ? *reinterpret_cast<const uint4*>(Hg + (q0 + r) * C::D + e) : uint4{0, 0, 0, 0};
      *reinterpret_cast<uint4*>(Ab + r * C::DPAD + e) = v;
    }
    __syncthreads();
    lane = opaque(lane);
    const int rb0 = wave * C::RPW, rh0 = wave * C::RPH;
    // y = h (C layout: rows = channels, columns = queries)
    f32x16 Y[C::RPW][NCB];
#pragma unroll
    for (int r = 0; r < C::RPW; ++r)
#pragma unroll
      for (int i = 0; i < NCB; ++i)
#pragma unroll
        for (int k = 0; k < 16; ++k)
          Y[r][i][k] = (float)Ab[(32 * i + (lane & 31)) * C::DPAD + 32 * (rb0 + r) + crow(k, lane)];
    for (int f0 = 0; f0 < A.F; f0 += C::FC) {
      f32x16 Hc[C::RPH][NCH];
#pragma unroll
      for (int r = 0; r < C::RPH; ++r)
#pragma unroll
        for (int j = 0; j < NCH; ++j) Hc[r][j] = zero16();
      gemm_rows<T, C::D / MM::KS, C::RPH, NCH, true>(wblock<C>(W1, f0 / 32 + rh0, 0, C::D), C::D, Ab, C::DPAD, 0, Hc,
                                                     lane);
#pragma unroll
      for (int r = 0; r < C::RPH; ++r)
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
          gelu_tile<C>(Hc[r][j], gtab);
          store_ct<T>(Hb + (32 * j) * C::HPAD + 32 * (rh0 + r), C::HPAD, Hc[r][j], lane);
        }
      __syncthreads();
      gemm_rows<T, C::FC / MM::KS, C::RPW, NCB, true>(wblock<C>(W2, rb0, f0 / MM::KS, A.F), A.F, Hb, C::HPAD, 0, Y,
                                                      lane);
      __syncthreads();
    }
    {
      float s[NCB];
#pragma unroll
      for (int i = 0; i < NCB; ++i) s[i] = 0.f;
#pragma unroll
      for (int r = 0; r < C::RPW; ++r) {
        float w[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) w[k] = A.w_head[32 * (rb0 + r) + crow(k, lane)];
#pragma unroll
        for (int i = 0; i < NCB; ++i)
#pragma unroll
          for (int k = 0; k < 16; ++k) s[i] += w[k] * Y[r][i][k];
      }
#pragma unroll
      for (int i = 0; i < NCB; ++i) {
        s[i] += __shfl_xor(s[i], 32);
        if (lane < 32) red[wave * C::BQ + 32 * i + lane] = s[i];
      }
    }
    __syncthreads();
    tid = opaque(tid);
    for (int t = tid; t < C::BQ; t += C::NT) {
      const int64_t q = q0 + t;
      if (q < q1) {
        float net = 0.f;
#pragma unroll
        for (int w = 0; w < C::NW; ++w) net += red[w * C::BQ + t];
        const Coords p{A.xyz[3 * q], A.xyz[3 * q + 1], A.xyz[3 * q + 2]};
        A.out[q] = analytic_sdf(p, A.prims) + A.net_scale * net;
      }
    }
    __syncthreads();
  }
}

hipError_t launch_local_head(const HeadArgs& a, hipStream_t s) {
  using C = CfgB256;
  if (a.N <= 0) return hipSuccess;
  constexpr int lds = C::LDS;
  static bool attr = false;
  const void* fn = reinterpret_cast<const void*>(&local_head_kernel<C>);
  if (!attr) {
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    attr = true;
  }
  int per_cu = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, local_head_kernel<C>, C::NT, lds);
  if (e != hipSuccess) return e;
  if (per_cu < 1) per_cu = 1;
  int64_t grid = (int64_t)dev_info().cus * per_cu;
  const int64_t tiles = (a.N + C::BQ - 1) / C::BQ;
  if (tiles < grid) grid = tiles;
  hipLaunchKernelGGL((local_head_kernel<C>), dim3((unsigned)grid), dim3(C::NT), lds, s, a);
  return hipGetLastError();
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

VDM_DEBUG_READER(debug_take_decode)

}  // namespace vdm
