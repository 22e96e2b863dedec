// Fused LayerNorm over the flattened [sum L, H] rows, and dtype conversions
// of the fp32 residual stream.
//
// 0h-n0.github.io Orca digest, implementation notes: LayerNorm statistics and
// scaling run as one fused kernel.  garden.houmin.site/infra/orca 3.1.2:
// LayerNorm mixes no tokens, so it runs on all rows of the batch at once.
//
// One workgroup per row: 128 threads (up to 16 per CU, so a 13B batch of 2176
// rows runs in one round), 256 for rows wider than 6144 (fewer registers per
// thread); the row stays in registers (16-byte
// loads, fully coalesced) between the mean pass, the centred variance pass
// and the normalise pass, so HBM sees one read of the fp32 row and one write
// of the output row: (4 + sizeof(T)) * H bytes per row.
#include "device.h"
#include "kernels.h"
#include "orca.h"

namespace orca {

constexpr int LN_MAX_VEC = 12;   // float4 per thread: H <= 12288 at 256 threads

template <int NT>
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x / 64, lane = threadIdx.x % 64;
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < NT / 64; ++i) t += red[i];
  return t;
}

// 4 consecutive elements of T as a float4 (8- or 16-byte access).
__device__ __forceinline__ float4 load4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 load4(const bf16* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return make_float4(bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y));
}
__device__ __forceinline__ void store4(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }
__device__ __forceinline__ void store4(bf16* p, float4 v) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
}

// NT threads, NV float4 per thread: the smallest instantiation that holds
// the row (registers beyond it would cut the workgroups resident per CU)
template <typename T, int NT, int NV>
__global__ __launch_bounds__(NT) void layernorm_kernel(const float* __restrict__ x,
                                                               const T* __restrict__ g,
                                                               const T* __restrict__ b,
                                                               T* __restrict__ out, int hidden,
                                                               float eps) {
  __shared__ float red[NT / 64];
  const int row = blockIdx.x;
  const float4* xr = reinterpret_cast<const float4*>(x + (size_t)row * hidden);
  const int nv = hidden / 4;
  // every load is issued before the first use, without branches (a chunk
  // past the row's end re-reads the last one and is zeroed): behind a
  // per-chunk branch each load waited for the one before.  Gamma and beta
  // are read with the row, so their latency hides behind the reductions.
  float4 v[NV], gg[NV], bb[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = min((int)threadIdx.x + i * NT, nv - 1);
    v[i] = xr[c];
    gg[i] = load4(g + c * 4);
    bb[i] = load4(b + c * 4);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    if ((int)threadIdx.x + i * NT >= nv) v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
  }
  const float mean = block_sum<NT>(s, red) / hidden;
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = threadIdx.x + i * NT;
    if (c < nv) {
      const float a = v[i].x - mean, e = v[i].y - mean, cc = v[i].z - mean, d = v[i].w - mean;
      q += (a * a + e * e) + (cc * cc + d * d);
    }
  }
  const float rstd = rsqrtf(block_sum<NT>(q, red) / hidden + eps);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = threadIdx.x + i * NT;
    if (c < nv) {
      float4 y;
      y.x = (v[i].x - mean) * rstd * gg[i].x + bb[i].x;
      y.y = (v[i].y - mean) * rstd * gg[i].y + bb[i].y;
      y.z = (v[i].z - mean) * rstd * gg[i].z + bb[i].z;
      y.w = (v[i].w - mean) * rstd * gg[i].w + bb[i].w;
      store4(out + (size_t)row * hidden + c * 4, y);
    }
  }
}

// Few-rows Linear with the residual epilogue, fused with the LayerNorm that
// follows it: one workgroup per row adds the row's fp32 split-K partial
// planes (in plane order) and the bias to the residual, exactly as the
// split-K reduce does, writes the new residual, and normalises it.  Saves
// the separate reduce launch (a tiny kernel costs ~4-5 us whatever it does).
// NT threads with NV float4 chunks each cover the row; every load of a
// chunk is issued before its first use.
template <int NT, int NV>
__global__ __launch_bounds__(NT) void reduce_resid_ln_kernel(
    const float* __restrict__ part, int splits, const bf16* __restrict__ bias,
    float* __restrict__ resid, int rows, int hidden, const bf16* __restrict__ g,
    const bf16* __restrict__ b, bf16* __restrict__ out, float eps) {
  __shared__ float red[NT / 64];
  const int row = blockIdx.x;
  const int nv = hidden / 4;
  const size_t plane = (size_t)rows * hidden, rbase = (size_t)row * hidden;
  float4 x[NV], v[NV], bi[NV], gg[NV], bb[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = min((int)threadIdx.x + i * NT, nv - 1);
    x[i] = *reinterpret_cast<const float4*>(resid + rbase + c * 4);
    v[i] = *reinterpret_cast<const float4*>(part + rbase + c * 4);
    bi[i] = load4(bias + c * 4);
    gg[i] = load4(g + c * 4);
    bb[i] = load4(b + c * 4);
  }
  for (int s0 = 1; s0 < splits; s0 += 4) {
    float4 t[4][NV];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int c = min((int)threadIdx.x + i * NT, nv - 1);
        t[u][i] = *reinterpret_cast<const float4*>(part + min(s0 + u, splits - 1) * plane +
                                                   rbase + c * 4);
      }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool on = s0 + u < splits;   // a select: behind a branch the load sinks into it
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        v[i].x += on ? t[u][i].x : 0.f; v[i].y += on ? t[u][i].y : 0.f;
        v[i].z += on ? t[u][i].z : 0.f; v[i].w += on ? t[u][i].w : 0.f;
      }
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = threadIdx.x + i * NT;
    x[i] = make_float4(x[i].x + (v[i].x + bi[i].x), x[i].y + (v[i].y + bi[i].y),
                       x[i].z + (v[i].z + bi[i].z), x[i].w + (v[i].w + bi[i].w));
    if (c < nv) {
      *reinterpret_cast<float4*>(resid + rbase + c * 4) = x[i];
      s += (x[i].x + x[i].y) + (x[i].z + x[i].w);
    }
  }
  const float mean = block_sum<NT>(s, red) / hidden;
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = threadIdx.x + i * NT;
    if (c < nv) {
      const float a = x[i].x - mean, e = x[i].y - mean, cc = x[i].z - mean, d = x[i].w - mean;
      q += (a * a + e * e) + (cc * cc + d * d);
    }
  }
  const float rstd = rsqrtf(block_sum<NT>(q, red) / hidden + eps);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = threadIdx.x + i * NT;
    if (c < nv) {
      float4 y;
      y.x = (x[i].x - mean) * rstd * gg[i].x + bb[i].x;
      y.y = (x[i].y - mean) * rstd * gg[i].y + bb[i].y;
      y.z = (x[i].z - mean) * rstd * gg[i].z + bb[i].z;
      y.w = (x[i].w - mean) * rstd * gg[i].w + bb[i].w;
      store4(out + rbase + c * 4, y);
    }
  }
}

template <typename T>
__global__ void to_f32_kernel(const T* __restrict__ in, float* __restrict__ out, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    out[i] = load_f32(in + i);
}

template <typename T>
__global__ void from_f32_kernel(const float* __restrict__ in, T* __restrict__ out, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    store_f32(out + i, in[i]);
}

template <typename T>
static void launch_ln_typed(const float* x, const void* g, const void* b, void* out, int rows,
                            int hidden, float eps, hipStream_t s) {
  const int v4 = hidden / 4;
#define ORCA_LN(NT, NV)                                                                      \
  hipLaunchKernelGGL((layernorm_kernel<T, NT, NV>), dim3(rows), dim3(NT), 0, s, x,           \
                     (const T*)g, (const T*)b, (T*)out, hidden, eps)
  if (v4 <= 128 * 2) ORCA_LN(128, 2);
  else if (v4 <= 128 * 4) ORCA_LN(128, 4);
  else if (v4 <= 128 * 6) ORCA_LN(128, 6);
  else if (v4 <= 128 * 8) ORCA_LN(128, 8);
  else if (v4 <= 128 * 10) ORCA_LN(128, 10);
  else if (v4 <= 128 * 12) ORCA_LN(128, 12);
  else if (v4 <= 256 * 8) ORCA_LN(256, 8);
  else if (v4 <= 256 * 10) ORCA_LN(256, 10);
  else ORCA_LN(256, LN_MAX_VEC);
#undef ORCA_LN
}

hipError_t launch_layernorm(int dtype, const float* x, const void* g, const void* b, void* out,
                            int rows, int hidden, float eps, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (dtype == ORCA_BF16) launch_ln_typed<bf16>(x, g, b, out, rows, hidden, eps, s);
  else launch_ln_typed<float>(x, g, b, out, rows, hidden, eps, s);
  return hipGetLastError();
}

static dim3 grid_for(int64_t n) {
  int64_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  return dim3((unsigned)(blocks > 0 ? blocks : 1));
}

hipError_t launch_reduce_resid_ln(const float* part, int splits, const void* bias, float* resid,
                                  int rows, int hidden, const void* g, const void* b, void* out,
                                  float eps, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const int v4 = hidden / 4;
  if (hidden % 4 != 0 || splits < 1) return hipErrorNotSupported;
#define ORCA_RRLN(NT, NV)                                                                     \
  hipLaunchKernelGGL((reduce_resid_ln_kernel<NT, NV>), dim3(rows), dim3(NT), 0, s, part, splits, \
                     (const bf16*)bias, resid, rows, hidden, (const bf16*)g, (const bf16*)b,  \
                     (bf16*)out, eps)
  if (v4 <= 256 * 2) ORCA_RRLN(256, 2);
  else if (v4 <= 512 * 2) ORCA_RRLN(512, 2);
  else if (v4 <= 640 * 2) ORCA_RRLN(640, 2);
  else if (v4 <= 768 * 2) ORCA_RRLN(768, 2);
  else if (v4 <= 1024 * 2) ORCA_RRLN(1024, 2);
  else if (v4 <= 768 * 4) ORCA_RRLN(768, 4);
  else return hipErrorNotSupported;   // (1024 x 4 would spill registers)
#undef ORCA_RRLN
  return hipGetLastError();
}

hipError_t launch_to_f32(int dtype, const void* in, float* out, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (dtype == ORCA_BF16)
    hipLaunchKernelGGL(to_f32_kernel<bf16>, grid_for(n), dim3(256), 0, s, (const bf16*)in, out, n);
  else
    hipLaunchKernelGGL(to_f32_kernel<float>, grid_for(n), dim3(256), 0, s, (const float*)in, out, n);
  return hipGetLastError();
}

hipError_t launch_from_f32(int dtype, const float* in, void* out, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (dtype == ORCA_BF16)
    hipLaunchKernelGGL(from_f32_kernel<bf16>, grid_for(n), dim3(256), 0, s, in, (bf16*)out, n);
  else
    hipLaunchKernelGGL(from_f32_kernel<float>, grid_for(n), dim3(256), 0, s, in, (float*)out, n);
  return hipGetLastError();
}

}  // namespace orca
