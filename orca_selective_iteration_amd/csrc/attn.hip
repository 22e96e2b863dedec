// Split attention: every request attends separately over its own K/V.
//
// garden.houmin.site/infra/orca 3.1.2: attention cannot be batched across
// requests (each request has its own keys, mask and cache), so the [sum L,
// 3H] QKV output is split per request, attention runs per request, and the
// outputs are merged back into [sum L, H]; splitting costs no weight traffic
// because attention reads no parameters.  0h-n0.github.io digest: attention
// is memory-bound.  estelledc.github.io notes, pitfalls: the K/V state, the
// position offset and the mask must line up per request.
//
// Split-KV path (increment rows, and every row of an fp32 model).  One
// query row q at absolute position p = kv_len + j sees keys 0..p of its
// request.  The keys are cut into work items of at most SPLIT_CHUNK keys;
// a 256-thread workgroup takes one (item, head).  Inside a wave, groups of
// LPK = d / (16 / sizeof(T)) lanes share one key: each lane loads 16 bytes
// of the key row and of the value row (so a wave reads 64 x 16 contiguous
// bytes per instruction), the partial dot products are summed with DPP row
// operations, and an online softmax (base 2, running max m and sum l per
// lane group) accumulates the value rows.  Four keys per lane group are in
// flight per loop trip.  The lane groups, then the four waves, are merged
// through shuffles and LDS into one (m, l, o[d]) partial per item; a second
// kernel merges the partials of a row and writes o at the row's own offset
// (the merge is index arithmetic: no copy).
//
// HBM traffic of the split path per (row, head): 2 * keys * d * sizeof(T)
// bytes of K and V, read once.
#include <math.h>

#include "device.h"
#include "kernels.h"
#include "orca.h"

namespace orca {

constexpr float LOG2E = 1.4426950408889634f;
constexpr float NEG_BIG = -1.0e30f;

template <typename T, int D>
__global__ __launch_bounds__(256) void attn_split_kernel(AttnArgs a) {
  constexpr int VEC = Vec16<T>::N;
  constexpr int LPK = D / VEC;       // lanes per key
  constexpr int KPW = 64 / LPK;      // keys per wave per load
  constexpr int NW = 4;
  constexpr int U = 4;
  constexpr int STRIDE = NW * KPW;   // keys per workgroup per load
  __shared__ float s_o[NW][D];
  __shared__ float s_ml[NW][2];

  const int item = blockIdx.x, h = blockIdx.y;
  const SplitItem it = a.items[item];
  const DevReq rq = a.reqs[it.req];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int e = lane % LPK, g = lane / LPK;
  const size_t H = (size_t)a.hidden;

  float q[VEC];
  Vec16<T>::unpack(*reinterpret_cast<const uint4*>((const T*)a.q + (size_t)it.row * H + h * D +
                                                   e * VEC),
                   q);
  const float sc = LOG2E / sqrtf((float)D);
#pragma unroll
  for (int v = 0; v < VEC; ++v) q[v] *= sc;

  const size_t head_base = ((size_t)h * a.cap + (size_t)rq.kv_base) * D + e * VEC;
  const T* kb = (const T*)a.k_pool + head_base;
  const T* vb = (const T*)a.v_pool + head_base;

  float m = NEG_BIG, l = 0.f, acc[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) acc[v] = 0.f;

  for (int base = it.c0 + w * KPW; base < it.c1; base += U * STRIDE) {
    uint4 kr[U], vr[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int key = base + g + u * STRIDE;
      ok[u] = key < it.c1;
      kr[u] = make_uint4(0, 0, 0, 0);
      vr[u] = make_uint4(0, 0, 0, 0);
      if (ok[u]) {
        kr[u] = *reinterpret_cast<const uint4*>(kb + (size_t)key * D);
        vr[u] = *reinterpret_cast<const uint4*>(vb + (size_t)key * D);
      }
    }
    float s[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kf[VEC];
      Vec16<T>::unpack(kr[u], kf);
      float p = 0.f;
#pragma unroll
      for (int v = 0; v < VEC; ++v) p = fmaf(q[v], kf[v], p);
      s[u] = group_sum<LPK>(p);
    }
    float mx = m;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (ok[u]) mx = fmaxf(mx, s[u]);
    const float corr = exp2f(m - mx);
    l *= corr;
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[v] *= corr;
    m = mx;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float p = ok[u] ? exp2f(s[u] - m) : 0.f;
      l += p;
      float vf[VEC];
      Vec16<T>::unpack(vr[u], vf);
#pragma unroll
      for (int v = 0; v < VEC; ++v) acc[v] = fmaf(p, vf[v], acc[v]);
    }
  }

  // merge the lane groups of the wave (lanes with equal e)
#pragma unroll
  for (int off = LPK; off < 64; off <<= 1) {
    const float m2 = __shfl_xor(m, off), l2 = __shfl_xor(l, off);
    const float mx = fmaxf(m, m2), c1 = exp2f(m - mx), c2 = exp2f(m2 - mx);
    l = l * c1 + l2 * c2;
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[v] = acc[v] * c1 + __shfl_xor(acc[v], off) * c2;
    m = mx;
  }
  if (g == 0) {
#pragma unroll
    for (int v = 0; v < VEC; ++v) s_o[w][e * VEC + v] = acc[v];
    if (e == 0) {
      s_ml[w][0] = m;
      s_ml[w][1] = l;
    }
  }
  __syncthreads();
  // merge the waves; one thread per output element
  for (int t = threadIdx.x; t < D; t += blockDim.x) {
    float mx = NEG_BIG;
#pragma unroll
    for (int i = 0; i < NW; ++i) mx = fmaxf(mx, s_ml[i][0]);
    float lt = 0.f, ot = 0.f;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const float c = exp2f(s_ml[i][0] - mx);
      lt += s_ml[i][1] * c;
      ot += s_o[i][t] * c;
    }
    const size_t pi = (size_t)item * a.heads + h;
    a.part_o[pi * D + t] = ot;
    if (t == 0) {
      a.part_ml[pi * 2 + 0] = mx;
      a.part_ml[pi * 2 + 1] = lt;
    }
  }
}

template <typename T, int D>
__global__ __launch_bounds__(128) void attn_combine_kernel(AttnArgs a) {
  const SplitRow sr = a.srows[blockIdx.x];
  const int h = blockIdx.y;
  for (int t = threadIdx.x; t < D; t += blockDim.x) {
    float mx = NEG_BIG;
    for (int i = 0; i < sr.item_count; ++i)
      mx = fmaxf(mx, a.part_ml[((size_t)(sr.item_begin + i) * a.heads + h) * 2]);
    float lt = 0.f, ot = 0.f;
    for (int i = 0; i < sr.item_count; ++i) {
      const size_t pi = (size_t)(sr.item_begin + i) * a.heads + h;
      const float c = exp2f(a.part_ml[pi * 2] - mx);
      lt += a.part_ml[pi * 2 + 1] * c;
      ot += a.part_o[pi * D + t] * c;
    }
    store_f32((T*)a.o + (size_t)sr.row * a.hidden + h * D + t, ot / lt);
  }
}

template <typename T, int D>
static void launch_split(const AttnArgs& a, hipStream_t s) {
  if (a.n_items == 0) return;
  hipLaunchKernelGGL((attn_split_kernel<T, D>), dim3(a.n_items, a.heads), dim3(256), 0, s, a);
  hipLaunchKernelGGL((attn_combine_kernel<T, D>), dim3(a.n_srows, a.heads), dim3(D < 128 ? D : 128),
                     0, s, a);
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  if (a.dtype == ORCA_BF16) {
    switch (a.head_dim) {
      case 64: launch_split<bf16, 64>(a, s); break;
      case 128: launch_split<bf16, 128>(a, s); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (a.head_dim) {
      case 16: launch_split<float, 16>(a, s); break;
      case 32: launch_split<float, 32>(a, s); break;
      case 64: launch_split<float, 64>(a, s); break;
      case 128: launch_split<float, 128>(a, s); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

}  // namespace orca
