// Per-shape preparation kernels: key/value projection (K = Z Wk^T, V = Z Wv^T),
// repacking of K/V into the tile layout the decoder streams, and the standalone
// embedding + Q projection.
//
// The vecset decoder of the FlashVDM pages (aipaper.cc summary, section 3)
// projects the latent tokens once per shape for cross-attention; these are the
// one-time steps before the per-query decode.
#include "vdm_device.hpp"

namespace vdm {

// ------------------------------------------------------------------ K/V packing
// The decoder's token loop reads, per 32-token tile t and head h, a run of 32
// elements per lane l (64 lanes): exactly the lane's MFMA operands.
//   K run, element e: A operand of S^T = K_h Q_h^T, step ks = e / KW, slot v = e % KW:
//       K[32t + l%32][64h + KS*ks + KW*(l/32) + v]
//   V run, element e: A operand of O^T += V_h^T P^T, row block db = e / 16, step
//       ps = (e % 16) / KW, slot v = e % KW:
//       V[32t + perm_key(KS*ps + KW*(l/32) + v)][64h + 32db + l%32]
// The runs are stored in 16-byte chunks, chunk-major: chunk c of all 64 lanes
// is one contiguous 1 KB (lane l at byte 16 l), so each 16-byte-per-lane load
// instruction of the decoder reads a contiguous 1 KB. A lane-major layout (each
// lane's run contiguous) makes every such load touch 4 KB and halves the
// vector-memory throughput. Tokens past M are zero.

// A batch of shapes runs on the second grid dimension: shape blockIdx.y reads K
// and V at byte offset y * in_stride and writes Kp and Vt at y * out_stride.
template <typename T>
__global__ void pack_kv_kernel(const T* __restrict__ K, const T* __restrict__ V, int M, int D, int Mpad,
                               T* __restrict__ Kp, T* __restrict__ Vt, int64_t in_stride, int64_t out_stride) {
  using MM = Mma<T>;
  constexpr int EPC = 16 / (int)sizeof(T);  // elements per 16-byte chunk
  K = reinterpret_cast<const T*>((const char*)K + blockIdx.y * in_stride);
  Kp = reinterpret_cast<T*>((char*)Kp + blockIdx.y * out_stride);
  if (Vt) {
    V = reinterpret_cast<const T*>((const char*)V + blockIdx.y * in_stride);
    Vt = reinterpret_cast<T*>((char*)Vt + blockIdx.y * out_stride);
  }
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n = (int64_t)Mpad * D;
  if (i >= n) return;
  const int64_t t = i / (32 * D);
  const int rem = (int)(i - t * 32 * D);
  const int h = rem / 2048, c = (rem % 2048) / (64 * EPC), l = (rem % (64 * EPC)) / EPC;
  const int e = c * EPC + rem % EPC;
  const int r = l & 31, half = l >> 5;
  {
    const int ks = e / MM::KW, v = e % MM::KW;
    const int64_t m = 32 * t + r;
    Kp[i] = m < M ? K[m * D + 64 * h + MM::KS * ks + MM::KW * half + v] : to_t<T>(0.f);
  }
  if (Vt) {
    const int db = e / 16, f = e % 16, ps = f / MM::KW, v = f % MM::KW;
    const int64_t m = 32 * t + perm_key<T>(MM::KS * ps + MM::KW * half + v);
    Vt[i] = m < M ? V[m * D + 64 * h + 32 * db + r] : to_t<T>(0.f);
  }
}

// ------------------------------------------------------------------ weight packing
// The decoder epilogue's A operands (rows of Wo, W1, W2) as contiguous 1 KB
// fragment blocks: one 16-byte-per-lane load per MFMA step (bf16 only).
__global__ void pack_w_kernel(const bf16* __restrict__ W, int rows, int cols, bf16* __restrict__ Wp) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // 16-byte chunk
  const int64_t n = (int64_t)rows * cols / 8;
  if (c >= n) return;
  const int nks = cols / 16;
  const int l = (int)(c % 64);
  const int64_t blk = c / 64;
  const int rb = (int)(blk / nks), ks = (int)(blk % nks);
  const int64_t src = (int64_t)(32 * rb + (l & 31)) * cols + 16 * ks + 8 * (l >> 5);
  reinterpret_cast<uint4*>(Wp)[c] = *reinterpret_cast<const uint4*>(W + src);
}

hipError_t launch_pack_w(const void* W, int rows, int cols, void* Wp, hipStream_t s) {
  const int64_t n = (int64_t)rows * cols / 8;
  const int bs = 256;
  hipLaunchKernelGGL(pack_w_kernel, dim3((unsigned)((n + bs - 1) / bs)), dim3(bs), 0, s, (const bf16*)W, rows, cols,
                     (bf16*)Wp);
  return hipGetLastError();
}

hipError_t launch_pack_kv(int dtype, const void* K, const void* V, int M, int D, int Mpad, void* Kp,
                          void* Vt, hipStream_t s, int B, int64_t in_stride, int64_t out_stride) {
  const int64_t n = (int64_t)Mpad * D;
  const int bs = 256;
  const dim3 g((unsigned)((n + bs - 1) / bs), (unsigned)B);
  if (dtype == VDM_BF16)
    hipLaunchKernelGGL(pack_kv_kernel<bf16>, g, dim3(bs), 0, s, (const bf16*)K, (const bf16*)V, M, D, Mpad,
                       (bf16*)Kp, (bf16*)Vt, in_stride, out_stride);
  else
    hipLaunchKernelGGL(pack_kv_kernel<float>, g, dim3(bs), 0, s, (const float*)K, (const float*)V, M, D, Mpad,
                       (float*)Kp, (float*)Vt, in_stride, out_stride);
  return hipGetLastError();
}

// kmax[h] = max over tokens of the Euclidean norm of head h's 64 key columns
// (float32; norms are non-negative, so their bit patterns order like integers).
// Thread i takes token i / H, head i % H (16-byte loads); the lanes of a wave that
// share a head reduce first, so each wave issues H atomics. H divides 64. A batch
// of shapes runs on the second grid dimension (K and kmax at byte strides).
template <typename T>
__global__ void key_norms_kernel(const T* __restrict__ K, int M, int H, float* kmax, int64_t k_stride,
                                 int64_t kmax_stride) {
  constexpr int EPC = 16 / (int)sizeof(T);
  K = reinterpret_cast<const T*>((const char*)K + blockIdx.y * k_stride);
  kmax = reinterpret_cast<float*>((char*)kmax + blockIdx.y * kmax_stride);
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int h = (int)(i % H);
  float s = 0.f;
  if (i < (int64_t)M * H) {
    const uint4* k = reinterpret_cast<const uint4*>(K + (i / H) * 64 * H + 64 * h);
#pragma unroll
    for (int c = 0; c < 64 / EPC; ++c) {
      const uint4 u = k[c];
      const T* x = reinterpret_cast<const T*>(&u);
#pragma unroll
      for (int e = 0; e < EPC; ++e) s += to_f(x[e]) * to_f(x[e]);
    }
  }
  float n = sqrtf(s);
  for (int o = 32; o >= H; o >>= 1) n = fmaxf(n, __shfl_xor(n, o));
  if ((threadIdx.x & 63) < H) atomicMax(reinterpret_cast<unsigned*>(kmax + h), __float_as_uint(n));
}

hipError_t launch_key_norms(int dtype, const void* K, int M, int H, float* kmax, hipStream_t s, int B,
                            int64_t k_stride, int64_t kmax_stride) {
  const int64_t n = (int64_t)M * H;
  const dim3 g((unsigned)((n + 255) / 256), (unsigned)B);
  if (dtype == VDM_BF16)
    hipLaunchKernelGGL(key_norms_kernel<bf16>, g, dim3(256), 0, s, (const bf16*)K, M, H, kmax, k_stride, kmax_stride);
  else
    hipLaunchKernelGGL(key_norms_kernel<float>, g, dim3(256), 0, s, (const float*)K, M, H, kmax, k_stride,
                       kmax_stride);
  return hipGetLastError();
}

// ------------------------------------------------------------------ K/V projection
// C^T[n][m] = sum_k W[n][k] Z[m][k] on MFMA; block tile 64 tokens x 64 outputs,
// one 32x32 tile per wave; blockIdx.z selects K (Wk) or V (Wv).

template <typename T>
__global__ __launch_bounds__(256) void project_kv_kernel(const T* __restrict__ Z, const T* __restrict__ Wk,
                                                         const T* __restrict__ Wv, int M, int D,
                                                         T* __restrict__ K, T* __restrict__ V) {
  using MM = Mma<T>;
  const T* W = blockIdx.z == 0 ? Wk : Wv;
  T* C = blockIdx.z == 0 ? K : V;
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int m0 = blockIdx.x * 64 + 32 * (wave & 1);
  const int n0 = blockIdx.y * 64 + 32 * (wave >> 1);
  const int mrow = min(m0 + (lane & 31), M - 1);  // clamp reads of the ragged last tile
  const T* zb = Z + (int64_t)mrow * D + MM::KW * (lane >> 5);
  const T* wb = W + (int64_t)(n0 + (lane & 31)) * D + MM::KW * (lane >> 5);
  f32x16 acc = zero16();
  for (int k = 0; k < D; k += MM::KS) {
    const auto a = *reinterpret_cast<const typename MM::frag*>(wb + k);
    const auto b = *reinterpret_cast<const typename MM::frag*>(zb + k);
    acc = MM::mma(a, b, acc);
  }
  const int m = m0 + (lane & 31);
  if (m < M) store_ct_row<T>(C + (int64_t)m * D + n0, acc, lane);
}

hipError_t launch_project_kv(int dtype, const void* Z, const void* Wk, const void* Wv, int M, int D, void* K,
                             void* V, hipStream_t s) {
  const dim3 g((M + 63) / 64, D / 64, 2);
  if (dtype == VDM_BF16)
    hipLaunchKernelGGL(project_kv_kernel<bf16>, g, dim3(256), 0, s, (const bf16*)Z, (const bf16*)Wk,
                       (const bf16*)Wv, M, D, (bf16*)K, (bf16*)V);
  else
    hipLaunchKernelGGL(project_kv_kernel<float>, g, dim3(256), 0, s, (const float*)Z, (const float*)Wk,
                       (const float*)Wv, M, D, (float*)K, (float*)V);
  return hipGetLastError();
}

// ------------------------------------------------------------------ embedding + Q projection

constexpr int EMB_BQ = 128;
constexpr int EMB_NT = 256;

template <typename T, int D>
__global__ __launch_bounds__(EMB_NT) void embed_kernel(QuerySrc qs, int64_t N, const T* __restrict__ Wq,
                                                       T* __restrict__ Q) {
  extern __shared__ __align__(16) char lds[];
  using L = EmbedLds<T, EMB_BQ, D>;
  const int64_t q0 = (int64_t)blockIdx.x * EMB_BQ;
  const int64_t q1 = min(q0 + EMB_BQ, N);
  embed_qproj<T, EMB_BQ, D, EMB_NT>(qs, q0, q1, Wq, lds, threadIdx.x);
  const T* Qs = reinterpret_cast<const T*>(lds + L::QS);
  constexpr int CH = D * (int)sizeof(T) / 16;  // 16-byte chunks per row
  for (int c = threadIdx.x; c < EMB_BQ * CH; c += EMB_NT) {
    const int qi = c / CH, ch = c % CH;
    if (q0 + qi < q1) {
      const int e = ch * 16 / (int)sizeof(T);
      *reinterpret_cast<uint4*>(Q + (q0 + qi) * D + e) = *reinterpret_cast<const uint4*>(Qs + qi * L::DPAD + e);
    }
  }
}

template <typename T, int D>
static hipError_t embed_t(const QuerySrc& qs, int64_t N, const void* Wq, void* Q, hipStream_t s) {
  using L = EmbedLds<T, EMB_BQ, D>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&embed_kernel<T, D>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, L::END);
  if (e != hipSuccess) return e;
  const dim3 g((unsigned)((N + EMB_BQ - 1) / EMB_BQ));
  hipLaunchKernelGGL((embed_kernel<T, D>), g, dim3(EMB_NT), L::END, s, qs, N, (const T*)Wq, (T*)Q);
  return hipGetLastError();
}

hipError_t launch_embed(int dtype, int D, const QuerySrc& qs, int64_t N, const void* Wq, void* Q,
                        hipStream_t s) {
  if (dtype == VDM_BF16) return D == 64 ? embed_t<bf16, 64>(qs, N, Wq, Q, s) : embed_t<bf16, 256>(qs, N, Wq, Q, s);
  return embed_t<float, 64>(qs, N, Wq, Q, s);
}

VDM_DEBUG_READER(debug_take_prep)

}  // namespace vdm
