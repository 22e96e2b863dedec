// The four Linear layers of the decoder block on the flattened [sum L, H]
// matrix, with their epilogues fused: bias; bias + GeLU; bias + residual add
// into the fp32 residual stream; and for the QKV projection the split of the
// 3H output columns into Q (kept as a [sum L, H] matrix) and K/V rows
// appended to each request's pool slots.
//
// garden.houmin.site/infra/orca 3.1.2: Linear mixes no tokens, so every
// request's rows form one [sum L, H] operand and the weights are read once
// for the whole batch; the fused QKV Linear yields 3H columns (H of Q, H of
// K, H of V); the split before attention and the K/V append are index
// arithmetic.  0h-n0.github.io digest, implementation notes: fused GeLU.
//
// bf16 path: MFMA (v_mfma_f32_32x32x16_bf16) with fp32 accumulation.
// Workgroup tile 128 x 128, K step 64, four waves each owning 64 x 64 of the
// output (2 x 2 MFMA tiles).  Both operands are K-contiguous in HBM (A is
// [M][K], W is [N][K]), loaded with 16-byte coalesced loads into registers,
// then into a double-buffered LDS stage padded by 16 bytes per row so the
// 16-byte fragment reads of a wave hit distinct banks.  One barrier per K
// step: the loads of step k+1 are in flight while step k runs on the MFMAs.
// The workgroup index is remapped so that each of the 8 XCDs (one L2 each)
// walks a contiguous range of tiles, M fastest, so the W column panel a tile
// needs is shared by the tiles resident on the same XCD.
//
// fp32 path: a plain LDS-tiled FMA kernel (64 x 64 tile) for fp32 models.
#include <math.h>

#include "device.h"
#include "kernels.h"
#include "orca.h"

namespace orca {

struct EpiParams {
  void* out;
  int ldo;
  QkvDest qkv;
};

__device__ __forceinline__ float gelu_tanh(float v) {
  // 0.5 v (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3)))  (Hendrycks & Gimpel)
  const float k0 = 0.7978845608028654f;
  return 0.5f * v * (1.f + tanhf(k0 * (v + 0.044715f * v * v * v)));
}

template <typename T, int EPI>
__device__ __forceinline__ void epi_store(const EpiParams& ep, int m, int n, float v) {
  if constexpr (EPI == ORCA_EPI_BIAS) {
    store_f32((T*)ep.out + (size_t)m * ep.ldo + n, v);
  } else if constexpr (EPI == ORCA_EPI_BIAS_GELU) {
    store_f32((T*)ep.out + (size_t)m * ep.ldo + n, gelu_tanh(v));
  } else if constexpr (EPI == ORCA_EPI_BIAS_RESID) {
    float* o = (float*)ep.out + (size_t)m * ep.ldo + n;
    *o += v;
  } else {
    const int H = ep.qkv.hidden;
    if (n < H) {
      store_f32((T*)ep.qkv.q_out + (size_t)m * H + n, v);
    } else {
      int c = n - H;
      T* pool = (T*)ep.qkv.k_pool;
      if (c >= H) {
        c -= H;
        pool = (T*)ep.qkv.v_pool;
      }
      const int d = ep.qkv.head_dim;
      const int h = c / d, dd = c - h * d;
      store_f32(pool + ((size_t)h * ep.qkv.cap + ep.qkv.row_dst[m]) * d + dd, v);
    }
  }
}

// ---------------------------------------------------------------- bf16 MFMA

constexpr int BM = 128, BN = 128, BK = 64, LDK = BK + 8;

__device__ __forceinline__ int xcd_remap(int b, int nblk) {
  const int q = nblk / 8, r = nblk % 8, xcd = b % 8, local = b / 8;
  return xcd < r ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
}

template <int EPI>
__global__ __launch_bounds__(256, 2) void gemm_bf16_kernel(const bf16* __restrict__ A,
                                                            const bf16* __restrict__ W,
                                                            const bf16* __restrict__ bias,
                                                            EpiParams ep, int M, int N, int K,
                                                            int tiles_m) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][BN * LDK];

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int tm = logical % tiles_m, tn = logical / tiles_m;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  const bf16* gA[4];
  const bf16* gB[4];
  int soff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i, row = c >> 3, ch = c & 7;
    const int am = min(tm * BM + row, M - 1), bn = min(tn * BN + row, N - 1);
    gA[i] = A + (size_t)am * K + ch * 8;
    gB[i] = W + (size_t)bn * K + ch * 8;
    soff[i] = row * LDK + ch * 8;
  }

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  uint4 ra[4], rb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ra[i] = *reinterpret_cast<const uint4*>(gA[i]);
    rb[i] = *reinterpret_cast<const uint4*>(gB[i]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    *reinterpret_cast<uint4*>(&sA[0][soff[i]]) = ra[i];
    *reinterpret_cast<uint4*>(&sB[0][soff[i]]) = rb[i];
  }
  __syncthreads();

  const int KT = K / BK;
  const int fr = lane & 31, fk = (lane >> 5) * 8;
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ra[i] = *reinterpret_cast<const uint4*>(gA[i] + (kt + 1) * BK);
        rb[i] = *reinterpret_cast<const uint4*>(gB[i] + (kt + 1) * BK);
      }
    }
    const uint16_t* a_base = &sA[cur][(wm * 64 + fr) * LDK + fk];
    const uint16_t* b_base = &sB[cur][(wn * 64 + fr) * LDK + fk];
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const bf16x8_t a0 = *reinterpret_cast<const bf16x8_t*>(a_base + ks * 16);
      const bf16x8_t a1 = *reinterpret_cast<const bf16x8_t*>(a_base + 32 * LDK + ks * 16);
      const bf16x8_t b0 = *reinterpret_cast<const bf16x8_t*>(b_base + ks * 16);
      const bf16x8_t b1 = *reinterpret_cast<const bf16x8_t*>(b_base + 32 * LDK + ks * 16);
      acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, acc[0][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b1, acc[0][1], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b0, acc[1][0], 0, 0, 0);
      acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, acc[1][1], 0, 0, 0);
    }
    if (kt + 1 < KT) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        *reinterpret_cast<uint4*>(&sA[cur ^ 1][soff[i]]) = ra[i];
        *reinterpret_cast<uint4*>(&sB[cur ^ 1][soff[i]]) = rb[i];
      }
    }
    __syncthreads();
  }

  // 32x32 accumulator layout: lane holds column lane%32 and rows
  // 8*(r/4) + 4*(lane/32) + r%4 for its 16 registers r.
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = tn * BN + wn * 64 + j * 32 + fr;
    if (n >= N) continue;
    const float bn = load_f32(bias + n);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = tm * BM + wm * 64 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        if (m < M) epi_store<bf16, EPI>(ep, m, n, acc[i][j][r] + bn);
      }
    }
  }
}

// ---------------------------------------------------------------- fp32 FMA

template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A,
                                                       const float* __restrict__ W,
                                                       const float* __restrict__ bias,
                                                       EpiParams ep, int M, int N, int K) {
  __shared__ float sA[16][64 + 4];
  __shared__ float sB[16][64 + 4];
  const int tm = blockIdx.y, tn = blockIdx.x, tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int lrow = tid >> 2, lk = (tid & 3) * 4;
  const int am = min(tm * 64 + lrow, M - 1), bn = min(tn * 64 + lrow, N - 1);
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
    const float4 va = *reinterpret_cast<const float4*>(A + (size_t)am * K + k0 + lk);
    const float4 vb = *reinterpret_cast<const float4*>(W + (size_t)bn * K + k0 + lk);
    sA[lk + 0][lrow] = va.x; sA[lk + 1][lrow] = va.y; sA[lk + 2][lrow] = va.z; sA[lk + 3][lrow] = va.w;
    sB[lk + 0][lrow] = vb.x; sB[lk + 1][lrow] = vb.y; sB[lk + 2][lrow] = vb.z; sB[lk + 3][lrow] = vb.w;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = sA[k][ty * 4 + i];
        b[i] = sB[k][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = tn * 64 + tx * 4 + j;
    if (n >= N) continue;
    const float bv = bias[n];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = tm * 64 + ty * 4 + i;
      if (m < M) epi_store<float, EPI>(ep, m, n, acc[i][j] + bv);
    }
  }
}

// ---------------------------------------------------------------- launcher

template <int EPI>
static void launch_typed(int dtype, const void* a, const void* w, const void* bias,
                         const EpiParams& ep, int m, int n, int k, hipStream_t s) {
  if (dtype == ORCA_BF16) {
    const int tiles_m = (m + BM - 1) / BM, tiles_n = (n + BN - 1) / BN;
    hipLaunchKernelGGL(gemm_bf16_kernel<EPI>, dim3(tiles_m * tiles_n), dim3(256), 0, s,
                       (const bf16*)a, (const bf16*)w, (const bf16*)bias, ep, m, n, k, tiles_m);
  } else {
    hipLaunchKernelGGL(gemm_f32_kernel<EPI>, dim3((n + 63) / 64, (m + 63) / 64), dim3(256), 0, s,
                       (const float*)a, (const float*)w, (const float*)bias, ep, m, n, k);
  }
}

hipError_t launch_linear(int dtype, int epilogue, const void* a, const void* w, const void* bias,
                         void* out, const QkvDest* qkv, int m, int n, int k, hipStream_t s) {
  if (m == 0) return hipSuccess;
  EpiParams ep{};
  ep.out = out;
  ep.ldo = n;
  if (qkv) ep.qkv = *qkv;
  switch (epilogue) {
    case ORCA_EPI_BIAS: launch_typed<ORCA_EPI_BIAS>(dtype, a, w, bias, ep, m, n, k, s); break;
    case ORCA_EPI_BIAS_GELU: launch_typed<ORCA_EPI_BIAS_GELU>(dtype, a, w, bias, ep, m, n, k, s); break;
    case ORCA_EPI_BIAS_RESID: launch_typed<ORCA_EPI_BIAS_RESID>(dtype, a, w, bias, ep, m, n, k, s); break;
    default: launch_typed<EPI_QKV>(dtype, a, w, bias, ep, m, n, k, s); break;
  }
  return hipGetLastError();
}

}  // namespace orca
