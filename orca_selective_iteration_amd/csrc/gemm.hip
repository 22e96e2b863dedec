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
// bf16 path: MFMA (v_mfma_f32_32x32x16_bf16) with fp32 accumulation, K step
// 64.  Both operands are K-contiguous in HBM (A is [M][K], W is [N][K]),
// loaded with 16-byte coalesced loads into registers, then into a
// double-buffered LDS stage padded by 16 bytes per row so the 16-byte
// fragment reads of a wave hit distinct banks; one barrier per K step.  The
// large Linear layers run on the four-wave kernel (256 x 256 or 256 x 192
// tiles, one wave per SIMD with its accumulators in the accumulation
// registers, the K step's traffic spread over its MFMAs); the eight-wave
// kernel (256 x 256 / 256 x 192 / 128 x 128 tiles) serves the few-rows
// split-K path and the fallbacks.  The workgroup index is remapped so that
// each of the 8 XCDs (one L2 each) walks a contiguous range of tiles, M
// fastest, so the W column panel a tile needs is shared by the tiles
// resident on the same XCD.
//
// fp32 path: a plain LDS-tiled FMA kernel (64 x 64 tile) for fp32 models.
#include <limits.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "device.h"
#include "kernels.h"
#include "orca.h"
#include "status.h"

namespace orca {

struct EpiParams {
  void* out;
  int ldo;
  QkvDest qkv;
};

__device__ __forceinline__ float gelu_tanh(float v) {
  // 0.5 v (1 + tanh(u)), u = sqrt(2/pi) (v + 0.044715 v^3)  (Hendrycks &
  // Gimpel).  With 1 + tanh(u) = 2 - 2 / (e + 1), e = exp(2u) = 2^(2u log2 e):
  // gelu = v - v / (e + 1), exact at both limits (e -> 0 gives 0, e -> inf
  // gives v).  The hardware exp2 and reciprocal (about 1 ulp each) replace
  // the correctly rounded division, which costs nine instructions.
  const float c1 = 2.f * 0.7978845608028654f * 1.4426950408889634f;   // 2 sqrt(2/pi) log2(e)
  const float c3 = c1 * 0.044715f;
  const float e = __builtin_amdgcn_exp2f(v * fmaf(c3, v * v, c1));
  return fmaf(-v, __builtin_amdgcn_rcpf(e + 1.f), v);
}

// One output column of a Linear layer, fixed per lane before the epilogue:
// where element (m, n) goes is col.ptr + m * col.stride, or for the K/V
// blocks of the QKV projection col.ptr + row_dst[m] * 2d (the pool slot,
// whose key row is followed by its value row).
template <typename T, int EPI>
struct EpiCol {
  T* ptr;
  size_t stride;
  bool slot;      // indexed by the row's pool slot instead of the row
  __device__ __forceinline__ EpiCol(const EpiParams& ep, int n) {
    slot = false;
    if constexpr (EPI == EPI_QKV) {
      const int H = ep.qkv.hidden, d = ep.qkv.head_dim;
      if (n < H) {
        ptr = (T*)ep.qkv.q_out + n;
        stride = H;
      } else {
        int c = n - H;
        T* pool = (T*)ep.qkv.kv_pool;
        if (c >= H) {
          c -= H;
          pool += d;   // the value row follows the key row
        }
        const int h = c / d, dd = c - h * d;
        ptr = pool + (size_t)h * ep.qkv.cap * 2 * d + dd;
        stride = 2 * d;
        slot = true;
      }
    } else {
      ptr = (T*)ep.out + n;
      stride = ep.ldo;
    }
  }
  // `row` is m, `dst` its pool slot (QKV only)
  __device__ __forceinline__ void store(int row, int dst, float v) const {
    T* p = ptr + (size_t)(slot ? dst : row) * stride;
    if constexpr (EPI == ORCA_EPI_BIAS || EPI == EPI_QKV || EPI == EPI_PARTIAL) {
      store_f32(p, v);
    } else if constexpr (EPI == ORCA_EPI_BIAS_GELU) {
      store_f32(p, gelu_tanh(v));
    } else {
      *reinterpret_cast<float*>(p) += v;
    }
  }
};

// ---------------------------------------------------------------- bf16 MFMA

constexpr int BK = 64, LDK = BK + 8;

__device__ __forceinline__ int xcd_remap(int b, int nblk) {
  const int q = nblk / 8, r = nblk % 8, xcd = b % 8, local = b / 8;
  return xcd < r ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
}

// Tile (tm, tn) of a launch-order index.  group <= 0: row tiles fastest
// (an XCD's concurrent workgroups cover every row tile of one or two column
// panels).  Otherwise the row tiles are taken in groups of `group`, and
// inside a group row tiles fastest, then column panels: an XCD's concurrent
// workgroups then share `group` A row panels and about 32 / group W column
// panels through its L2.
__device__ __forceinline__ void tile_of(int logical, int tiles_m, int ntiles, int group, int& tm,
                                        int& tn) {
  if (group <= 0 || group >= tiles_m) {
    tm = logical % tiles_m;
    tn = logical / tiles_m;
    return;
  }
  const int per_group = group * (ntiles / tiles_m);
  const int g = logical / per_group, idx = logical - g * per_group;
  const int gm = min(group, tiles_m - g * group);
  tm = g * group + idx % gm;
  tn = idx / gm;
}

// Which tiles a four-wave launch covers.  A launch takes the logical tiles
// tile_base .. tile_base + gridDim.x - 1 of a problem of ntiles tiles
// (tile_of's order), each over K steps [y * kt_per_split, ...) for
// blockIdx.y = y.  A data-parallel launch covers every tile over all of K;
// the split-K tail of a hybrid launch covers the last n_tail tiles with K
// split over grid.y, each split writing fp32 partial sums, tile-major.
struct TileMap {
  int tiles_m, ntiles, group;
  int tile_base, kt_per_split, n_tail;
  // > 0: a persistent launch of gridDim.x workgroups covers this many tiles
  // (from tile_base), each XCD a contiguous share of them, its workgroups
  // walking it in strides of one round; 0: one tile per workgroup
  int persist;
  // > 0: a main-and-helper tail, a tile's K steps (see sk_segment); 0: the
  // tail's K is split evenly over grid.y
  int sk_kt;
};

// Main-and-helper tail (a form of stream-K): gridDim.x = NUM_CU workgroups
// share the n_tail tail tiles.  Workgroup g < n_tail (logical) is tile g's
// main: K steps [0, x), x = kt_per_split.  The other gridDim.x - n_tail are
// helpers: helper h takes steps [x, sk_kt) of tiles h, h + helpers, ...
// Mains run the same K steps of neighbouring tiles at the same time, and so
// do the helpers, so an XCD's workgroups share A and W panels through its
// L2 as in a full round.  (Contiguous ranges of the tiles' K steps laid end
// to end balance exactly but leave every workgroup at its own K offset: on
// the 175B-layer FFN2 that read ~10 GB for the round and ran 0.3 ms slower
// than no tail.)  Tile t's partial sums: slot t (main), n_tail + t (helper).
__device__ __forceinline__ int sk_segments(const TileMap& m, int g) {
  const int helpers = gridDim.x - m.n_tail, h = g - m.n_tail;
  return g < m.n_tail ? 1 : (m.n_tail - h + helpers - 1) / helpers;
}
__device__ __forceinline__ void sk_segment(const TileMap& m, int g, int seg, int& tile, int& k0,
                                           int& kt, size_t& slot) {
  if (g < m.n_tail) {
    tile = g;
    k0 = 0;
    kt = m.kt_per_split;
    slot = g;
  } else {
    tile = g - m.n_tail + seg * (gridDim.x - m.n_tail);
    k0 = m.kt_per_split;
    kt = m.sk_kt - m.kt_per_split;
    slot = (size_t)m.n_tail + tile;
  }
}

// Workgroup tile (WGM*32*TI) x (WGN*32*TJ): a WGM x WGN grid of waves, each
// owning (32*TI) x (32*TJ) outputs as TI x TJ 32x32 MFMA accumulators.
template <int WGM, int WGN, int TI, int TJ>
struct TileCfg {
  static constexpr int NT = 64 * WGM * WGN;                    // threads
  static constexpr int BM = WGM * 32 * TI, BN = WGN * 32 * TJ;
  static constexpr int LA = BM * 8 / NT, LB = BN * 8 / NT;     // 16-byte loads per thread
  static_assert(LA * NT == BM * 8 && LB * NT == BN * 8, "tile not divisible by threads");
};

template <bool NT>
__device__ __forceinline__ uint4 load_w(const bf16* p) {
  if constexpr (NT) return load_nt16(p);
  else return *reinterpret_cast<const uint4*>(p);
}

// The epilogue of one wave's (32*TI) x (32*TJ) accumulators whose first
// row is m0 and first column n0.  32x32 accumulator layout: lane holds
// column lane%32 and rows 8*(r/4) + 4*(lane/32) + r%4 for its 16 registers r.
template <int EPI, int TI, int TJ, int RB = 16>
__device__ __forceinline__ void store_wave_tile(const f32x16_t (&acc)[TI][TJ],
                                                const bf16* __restrict__ bias,
                                                const EpiParams& ep, int M, int N, int m0,
                                                int n0, int lane) {
  using OutT = typename std::conditional<EPI == ORCA_EPI_BIAS_RESID || EPI == EPI_PARTIAL, float,
                                         bf16>::type;
  const int fr = lane & 31;
  float bn[TJ];
#pragma unroll
  for (int j = 0; j < TJ; ++j)
    bn[j] = EPI == EPI_PARTIAL ? 0.f : load_f32(bias + min(n0 + j * 32 + fr, N - 1));
  if constexpr (EPI == ORCA_EPI_BIAS_RESID) {
    // read-modify-write of the fp32 residual.  Element by element the
    // compiler keeps every read behind the previous write (it cannot prove
    // that they do not alias) and the epilogue becomes a chain of memory
    // round trips; so a wave whose tile lies inside the matrix issues RB
    // reads before their writes, addressed as a wave-uniform row base plus
    // one per-lane 32-bit offset (few registers: the kernels run close to
    // their register limit).  Edge waves, and RB = 0, take the element-wise
    // path.
    float* const out = static_cast<float*>(ep.out);
    int ldo = ep.ldo;
    // opaque to the optimiser: keeps the address arithmetic here instead of
    // hoisted above the K loop, where it would hold registers through it
    asm volatile("" : "+s"(ldo));
    if (RB > 0 && m0 + 32 * TI <= M && n0 + 32 * TJ <= N) {
      const uint32_t loff = ((uint32_t)((lane >> 5) * 4) * ldo + fr) * 4u;
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int r0 = 0; r0 < 16; r0 += (RB > 0 ? RB : 16)) {
            float old[RB > 0 ? RB : 1];
#pragma unroll
            for (int r = r0; r < r0 + RB; ++r) {
              const char* row = reinterpret_cast<const char*>(
                  out + (size_t)(m0 + i * 32 + (r >> 2) * 8 + (r & 3)) * ldo + n0 + j * 32);
              old[r - r0] = *reinterpret_cast<const float*>(row + loff);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int r = r0; r < r0 + RB; ++r) {
              char* row = reinterpret_cast<char*>(
                  out + (size_t)(m0 + i * 32 + (r >> 2) * 8 + (r & 3)) * ldo + n0 + j * 32);
              *reinterpret_cast<float*>(row + loff) = old[r - r0] + (acc[i][j][r] + bn[j]);
            }
          }
    } else {
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int n = n0 + j * 32 + fr;
        if (n >= N) continue;
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int m = m0 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
            if (m < M) out[(size_t)m * ldo + n] += acc[i][j][r] + bn[j];
          }
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < TI; ++i) {
    // the pool slots of the sixteen rows, read together before any write
    // (read one by one between the writes, each is a round trip; RB = 0
    // keeps that form, which needs fewer registers)
    int dst[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
      dst[r] = EPI == EPI_QKV && RB > 0 ? ep.qkv.row_dst[min(m, M - 1)] : 0;
    }
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int n = n0 + j * 32 + fr;
      if (n >= N) continue;
      const EpiCol<OutT, EPI> col(ep, n);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        if (m < M)
          col.store(m, EPI == EPI_QKV && RB == 0 ? ep.qkv.row_dst[m] : dst[r],
                    acc[i][j][r] + bn[j]);
      }
    }
  }
}

// The epilogue of a wave's (32*TI) x (32*TJ) accumulators computed
// transposed (W as the MFMA's first operand, so each accumulator holds
// C^T): for accumulator [i][j], lane l holds output row m0 + 32 i + l % 32,
// and its registers 4 q .. 4 q + 3 hold the four consecutive columns
// n0 + 32 j + 8 q + 4 (l / 32) + 0..3 of that row.  Each register group is
// one 8-byte (bf16) or 16-byte (fp32) access, a quarter of the element-wise
// stores, and the QKV pool slot is read once per row.  N is a multiple of
// 64, so a 32-column block is inside the matrix or outside it whole.
template <int EPI, int TI, int TJ>
__device__ __forceinline__ void store_wave_tile_t(const f32x16_t (&acc)[TI][TJ],
                                                  const bf16* __restrict__ bias,
                                                  const EpiParams& ep, int M, int N, int m0,
                                                  int n0, int lane) {
  const int mr = lane & 31, nh = (lane >> 5) * 4;
  float bq[TJ][4][4];
#pragma unroll
  for (int j = 0; j < TJ; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int n = min(n0 + 32 * j + 8 * q + nh, N - 4);
      const uint2 w = EPI == EPI_PARTIAL ? make_uint2(0u, 0u)
                                         : *reinterpret_cast<const uint2*>(bias + n);
      bq[j][q][0] = bf16_lo(w.x);
      bq[j][q][1] = bf16_hi(w.x);
      bq[j][q][2] = bf16_lo(w.y);
      bq[j][q][3] = bf16_hi(w.y);
    }
  if constexpr (EPI == ORCA_EPI_BIAS_RESID) {
    // fp32 read-modify-write.  The compiler cannot prove that the reads and
    // writes do not alias, so it keeps them in program order: each row
    // block's reads are issued before the previous block's writes, and one
    // memory latency is exposed per tile rather than per row block.
    float4 cur[TJ][4], nxt[TJ][4];
#define ORCA_RESID_READ(DST, I)                                                               \
  {                                                                                           \
    const float* row = static_cast<const float*>(ep.out) +                                    \
                       (size_t)min(m0 + 32 * (I) + mr, M - 1) * ep.ldo;                      \
    _Pragma("unroll") for (int j = 0; j < TJ; ++j)                                            \
        _Pragma("unroll") for (int q = 0; q < 4; ++q) DST[j][q] =                             \
            *reinterpret_cast<const float4*>(row + min(n0 + 32 * j + 8 * q + nh, N - 4));     \
  }
    ORCA_RESID_READ(cur, 0)
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      if (i + 1 < TI) ORCA_RESID_READ(nxt, i + 1)
      __builtin_amdgcn_sched_barrier(0);
      const int m = m0 + 32 * i + mr;
      float* const row = static_cast<float*>(ep.out) + (size_t)min(m, M - 1) * ep.ldo;
      if (m < M) {
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          if (n0 + 32 * j >= N) continue;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float4 v = cur[j][q];
            v.x += acc[i][j][4 * q] + bq[j][q][0];
            v.y += acc[i][j][4 * q + 1] + bq[j][q][1];
            v.z += acc[i][j][4 * q + 2] + bq[j][q][2];
            v.w += acc[i][j][4 * q + 3] + bq[j][q][3];
            *reinterpret_cast<float4*>(row + n0 + 32 * j + 8 * q + nh) = v;
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if (i + 1 < TI) {
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) cur[j][q] = nxt[j][q];
      }
    }
#undef ORCA_RESID_READ
    return;
  }
  // the QKV pool slots of the lane's rows, read before any write
  int slots[TI];
#pragma unroll
  for (int i = 0; i < TI; ++i)
    slots[i] = EPI == EPI_QKV ? ep.qkv.row_dst[min(m0 + 32 * i + mr, M - 1)] : 0;
#pragma unroll
  for (int i = 0; i < TI; ++i) {
    const int m = m0 + 32 * i + mr, slot = slots[i];
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      if (n0 + 32 * j >= N) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + 32 * j + 8 * q + nh;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = acc[i][j][4 * q + e] + bq[j][q][e];
          if constexpr (EPI == ORCA_EPI_BIAS_GELU) v[e] = gelu_tanh(v[e]);
        }
        if constexpr (EPI == EPI_PARTIAL) {
          *reinterpret_cast<float4*>(static_cast<float*>(ep.out) + (size_t)m * ep.ldo + n) =
              make_float4(v[0], v[1], v[2], v[3]);
        } else {
          // the four columns lie in one head of one block (d % 4 == 0)
          const EpiCol<bf16, EPI> col(ep, n);
          *reinterpret_cast<uint2*>(col.ptr + (size_t)(col.slot ? slot : m) * col.stride) =
              make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        }
      }
    }
  }
}

// STREAM_W: W is read by one row tile only (the few-rows path), so its
// loads carry the non-temporal hint; otherwise W panels are re-read by the
// other row tiles through L2 and load plainly.
template <int EPI, int WGM, int WGN, int TI, int TJ, bool PIPE, bool STREAM_W = false>
__global__ __launch_bounds__(64 * WGM * WGN, (WGM * WGN == 4 && TI * TJ <= 4) ? 2 : 1)
void gemm_bf16_kernel(const bf16* __restrict__ A, const bf16* __restrict__ W,
                      const bf16* __restrict__ bias, EpiParams ep, int M, int N, int K,
                      int tiles_m, int kt_per_split) {
  using C = TileCfg<WGM, WGN, TI, TJ>;
  // grid.y splits K: this workgroup sums K steps [k0, k0 + KT) (the whole
  // of K unless the epilogue writes fp32 partial sums)
  const int k0 = blockIdx.y * kt_per_split;
  const int KT = min(K / BK - k0, kt_per_split);
  A += (size_t)k0 * BK;
  W += (size_t)k0 * BK;
  if constexpr (EPI == EPI_PARTIAL) ep.out = static_cast<float*>(ep.out) + (size_t)blockIdx.y * M * N;
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][C::BM * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][C::BN * LDK];

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int tm = logical % tiles_m, tn = logical / tiles_m;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;

  const bf16* gA[C::LA];
  const bf16* gB[C::LB];
  int oA[C::LA], oB[C::LB];
#pragma unroll
  for (int i = 0; i < C::LA; ++i) {
    const int c = tid + C::NT * i, row = c >> 3, ch = c & 7;
    gA[i] = A + (size_t)min(tm * C::BM + row, M - 1) * K + ch * 8;
    oA[i] = row * LDK + ch * 8;
  }
#pragma unroll
  for (int i = 0; i < C::LB; ++i) {
    const int c = tid + C::NT * i, row = c >> 3, ch = c & 7;
    gB[i] = W + (size_t)min(tn * C::BN + row, N - 1) * K + ch * 8;
    oB[i] = row * LDK + ch * 8;
  }

  f32x16_t acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  uint4 ra[C::LA], rb[C::LB];
#pragma unroll
  for (int i = 0; i < C::LA; ++i) ra[i] = *reinterpret_cast<const uint4*>(gA[i]);
#pragma unroll
  for (int i = 0; i < C::LB; ++i) rb[i] = load_w<STREAM_W>(gB[i]);
#pragma unroll
  for (int i = 0; i < C::LA; ++i) *reinterpret_cast<uint4*>(&sA[0][oA[i]]) = ra[i];
#pragma unroll
  for (int i = 0; i < C::LB; ++i) *reinterpret_cast<uint4*>(&sB[0][oB[i]]) = rb[i];
  __syncthreads();

  const int fr = lane & 31, fk = (lane >> 5) * 8;
  const int a_off = (wm * 32 * TI + fr) * LDK + fk, b_off = (wn * 32 * TJ + fr) * LDK + fk;
  if constexpr (!PIPE) {
    for (int kt = 0; kt < KT; ++kt) {
      const int cur = kt & 1;
      // prefetch the next K step (the last trip re-reads the current one, so
      // the staging registers never sit behind a branch)
      const int kn = min(kt + 1, KT - 1) * BK;
#pragma unroll
      for (int i = 0; i < C::LA; ++i) ra[i] = *reinterpret_cast<const uint4*>(gA[i] + kn);
#pragma unroll
      for (int i = 0; i < C::LB; ++i) rb[i] = load_w<STREAM_W>(gB[i] + kn);
      __builtin_amdgcn_sched_barrier(0);
      const uint16_t* a_base = &sA[cur][a_off];
      const uint16_t* b_base = &sB[cur][b_off];
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        bf16x8_t a[TI], b[TJ];
#pragma unroll
        for (int i = 0; i < TI; ++i)
          a[i] = *reinterpret_cast<const bf16x8_t*>(a_base + i * 32 * LDK + ks * 16);
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          b[j] = *reinterpret_cast<const bf16x8_t*>(b_base + j * 32 * LDK + ks * 16);
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int j = 0; j < TJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < C::LA; ++i) *reinterpret_cast<uint4*>(&sA[cur ^ 1][oA[i]]) = ra[i];
#pragma unroll
      for (int i = 0; i < C::LB; ++i) *reinterpret_cast<uint4*>(&sB[cur ^ 1][oB[i]]) = rb[i];
      __syncthreads();
    }
  } else {
    // Two K steps in flight: at step kt the loads of step kt+2 are issued
    // into one register set while the other set (step kt+1, requested a
    // whole step earlier) is written to the LDS buffer freed by step kt-1.
    // The sets are vector values (not arrays) so they stay in registers.
    typedef uint32_t StageA __attribute__((ext_vector_type(4 * C::LA)));
    typedef uint32_t StageB __attribute__((ext_vector_type(4 * C::LB)));
    StageA pa0, pa1;
    StageB pb0, pb1;
#define ORCA_LOAD_STAGE(PA, PB, KOFF)                                                        \
  _Pragma("unroll") for (int i = 0; i < C::LA; ++i) {                                        \
    const uint4 t = *reinterpret_cast<const uint4*>(gA[i] + (KOFF));                         \
    PA[4 * i] = t.x; PA[4 * i + 1] = t.y; PA[4 * i + 2] = t.z; PA[4 * i + 3] = t.w;          \
  }                                                                                          \
  _Pragma("unroll") for (int i = 0; i < C::LB; ++i) {                                        \
    const uint4 t = load_w<STREAM_W>(gB[i] + (KOFF));                                        \
    PB[4 * i] = t.x; PB[4 * i + 1] = t.y; PB[4 * i + 2] = t.z; PB[4 * i + 3] = t.w;          \
  }
#define ORCA_STORE_STAGE(PA, PB, BUF)                                                        \
  _Pragma("unroll") for (int i = 0; i < C::LA; ++i)                                          \
      *reinterpret_cast<uint4*>(&sA[BUF][oA[i]]) =                                           \
          make_uint4(PA[4 * i], PA[4 * i + 1], PA[4 * i + 2], PA[4 * i + 3]);                \
  _Pragma("unroll") for (int i = 0; i < C::LB; ++i)                                          \
      *reinterpret_cast<uint4*>(&sB[BUF][oB[i]]) =                                           \
          make_uint4(PB[4 * i], PB[4 * i + 1], PB[4 * i + 2], PB[4 * i + 3]);
#define ORCA_GEMM_STEP(KT_, LA_, LB_, WA_, WB_)                                              \
  {                                                                                          \
    const int cur = (KT_) & 1;                                                               \
    ORCA_LOAD_STAGE(LA_, LB_, min((KT_) + 2, KT - 1) * BK)                                   \
    ORCA_STORE_STAGE(WA_, WB_, cur ^ 1)                                                      \
    __builtin_amdgcn_sched_barrier(0);                                                       \
    const uint16_t* a_base = &sA[cur][a_off];                                                \
    const uint16_t* b_base = &sB[cur][b_off];                                                \
    _Pragma("unroll") for (int ks = 0; ks < BK / 16; ++ks) {                                 \
      bf16x8_t a[TI], b[TJ];                                                                 \
      _Pragma("unroll") for (int i = 0; i < TI; ++i) a[i] =                                  \
          *reinterpret_cast<const bf16x8_t*>(a_base + i * 32 * LDK + ks * 16);               \
      _Pragma("unroll") for (int j = 0; j < TJ; ++j) b[j] =                                  \
          *reinterpret_cast<const bf16x8_t*>(b_base + j * 32 * LDK + ks * 16);               \
      _Pragma("unroll") for (int i = 0; i < TI; ++i)                                         \
          _Pragma("unroll") for (int j = 0; j < TJ; ++j) acc[i][j] =                         \
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);       \
    }                                                                                        \
    __syncthreads();                                                                         \
  }
    ORCA_LOAD_STAGE(pa1, pb1, min(1, KT - 1) * BK)
    // the launcher takes this path only for an even number of K steps
    for (int kt = 0; kt < KT; kt += 2) {
      ORCA_GEMM_STEP(kt, pa0, pb0, pa1, pb1)
      ORCA_GEMM_STEP(kt + 1, pa1, pb1, pa0, pb0)
    }
#undef ORCA_GEMM_STEP
#undef ORCA_LOAD_STAGE
#undef ORCA_STORE_STAGE
  }

  store_wave_tile<EPI, TI, TJ>(acc, bias, ep, M, N, tm * C::BM + wm * 32 * TI,
                               tn * C::BN + wn * 32 * TJ, lane);
}

// ------------------------------------------------- wave-specialised 256 x 256

// 256 x 256 tile with the work split by wave: eight MFMA waves (a 4 x 2 grid,
// 64 x 128 each, as in the tile above) only read LDS and issue MFMAs, and
// four loader waves move the K steps from global memory through registers
// into the double-buffered LDS stage.  A loader holds two K steps in
// registers, so a load has two whole steps to arrive before its data is
// written to LDS, and the MFMA waves never wait on global memory.  All
// twelve waves meet at one barrier per K step: after it the MFMA waves read
// the buffer written before it, while the loaders fill the other one.
// Needs an even number of K steps and element offsets below 2^31.
constexpr int WS_THREADS = 768, WS_LOADERS = 256;

template <int EPI>
__global__ __launch_bounds__(WS_THREADS, 1)
void gemm_ws_kernel(const bf16* __restrict__ A, const bf16* __restrict__ W,
                    const bf16* __restrict__ bias, EpiParams ep, int M, int N, int K,
                    int tiles_m) {
  constexpr int BM = 256, BN = 256, TI = 2, TJ = 4;
  constexpr int LD = BM * 8 / WS_LOADERS;   // 16-byte chunks per loader lane and operand
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][BN * LDK];

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int tm = logical % tiles_m, tn = logical / tiles_m;
  const int tid = threadIdx.x, lane = tid & 63;
  // wave-uniform role (a scalar branch: each path runs its own barriers)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int KT = K / BK;

  if (wave >= 8) {
    const int lt = tid - 8 * 64, ch = lt & 7;
    // byte offsets from the operand base (a uniform base plus a 32-bit
    // offset per load keeps the loader's addresses to one register each)
    uint32_t offA[LD], offB[LD];
#pragma unroll
    for (int i = 0; i < LD; ++i) {
      const int row = (lt >> 3) + 32 * i;
      offA[i] = (uint32_t)(min(tm * BM + row, M - 1) * K + ch * 8) * 2u;
      offB[i] = (uint32_t)(min(tn * BN + row, N - 1) * K + ch * 8) * 2u;
    }
    const int oL = (lt >> 3) * LDK + ch * 8;   // chunk i lands 32 rows further down
    typedef uint32_t Stage __attribute__((ext_vector_type(8 * LD)));
    Stage s0, s1;
#define ORCA_WS_LOAD(S, KS)                                                                   \
  {                                                                                           \
    const char* bA = reinterpret_cast<const char*>(A) + (size_t)(KS) * BK * 2;                \
    const char* bB = reinterpret_cast<const char*>(W) + (size_t)(KS) * BK * 2;                \
    _Pragma("unroll") for (int i = 0; i < LD; ++i) {                                          \
      const uint4 a = *reinterpret_cast<const uint4*>(bA + offA[i]);                          \
      S[4 * i] = a.x; S[4 * i + 1] = a.y; S[4 * i + 2] = a.z; S[4 * i + 3] = a.w;             \
    }                                                                                         \
    _Pragma("unroll") for (int i = 0; i < LD; ++i) {                                          \
      const uint4 b = *reinterpret_cast<const uint4*>(bB + offB[i]);                          \
      S[4 * LD + 4 * i] = b.x; S[4 * LD + 4 * i + 1] = b.y;                                   \
      S[4 * LD + 4 * i + 2] = b.z; S[4 * LD + 4 * i + 3] = b.w;                               \
    }                                                                                         \
  }
#define ORCA_WS_STORE(S, BUF)                                                                 \
  {                                                                                           \
    _Pragma("unroll") for (int i = 0; i < LD; ++i)                                            \
        *reinterpret_cast<uint4*>(&sA[BUF][oL + i * 32 * LDK]) =                              \
            make_uint4(S[4 * i], S[4 * i + 1], S[4 * i + 2], S[4 * i + 3]);                   \
    _Pragma("unroll") for (int i = 0; i < LD; ++i)                                            \
        *reinterpret_cast<uint4*>(&sB[BUF][oL + i * 32 * LDK]) =                              \
            make_uint4(S[4 * LD + 4 * i], S[4 * LD + 4 * i + 1], S[4 * LD + 4 * i + 2],       \
                       S[4 * LD + 4 * i + 3]);                                                \
  }
    ORCA_WS_LOAD(s0, 0)
    ORCA_WS_LOAD(s1, min(1, KT - 1))
    ORCA_WS_STORE(s0, 0)
    ORCA_WS_LOAD(s0, min(2, KT - 1))
    __syncthreads();
    // at the barrier ending step kt the buffer of step kt+1 is full; the
    // registers then take step kt+3 (clamped: the last trips re-read)
    for (int kt = 0; kt < KT; kt += 2) {
      ORCA_WS_STORE(s1, 1)
      ORCA_WS_LOAD(s1, min(kt + 3, KT - 1))
      __syncthreads();
      ORCA_WS_STORE(s0, 0)
      ORCA_WS_LOAD(s0, min(kt + 4, KT - 1))
      __syncthreads();
    }
#undef ORCA_WS_LOAD
#undef ORCA_WS_STORE
    return;
  }

  const int wm = wave >> 1, wn = wave & 1;
  const int fr = lane & 31, fk = (lane >> 5) * 8;
  const int a_off = (wm * 32 * TI + fr) * LDK + fk, b_off = (wn * 32 * TJ + fr) * LDK + fk;
  f32x16_t acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
#define ORCA_WS_COMPUTE(BUF)                                                                  \
  {                                                                                           \
    const uint16_t* a_base = &sA[BUF][a_off];                                                 \
    const uint16_t* b_base = &sB[BUF][b_off];                                                 \
    _Pragma("unroll") for (int ks = 0; ks < BK / 16; ++ks) {                                  \
      bf16x8_t a[TI], b[TJ];                                                                  \
      _Pragma("unroll") for (int i = 0; i < TI; ++i) a[i] =                                   \
          *reinterpret_cast<const bf16x8_t*>(a_base + i * 32 * LDK + ks * 16);                \
      _Pragma("unroll") for (int j = 0; j < TJ; ++j) b[j] =                                   \
          *reinterpret_cast<const bf16x8_t*>(b_base + j * 32 * LDK + ks * 16);                \
      _Pragma("unroll") for (int i = 0; i < TI; ++i)                                          \
          _Pragma("unroll") for (int j = 0; j < TJ; ++j) acc[i][j] =                          \
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);        \
    }                                                                                         \
  }
  __syncthreads();
  for (int kt = 0; kt < KT; kt += 2) {
    ORCA_WS_COMPUTE(0)
    __syncthreads();
    ORCA_WS_COMPUTE(1)
    __syncthreads();
  }
#undef ORCA_WS_COMPUTE
  // element by element (RB = 0): at 168 registers the batched residual
  // and pool-slot reads spill
  store_wave_tile<EPI, TI, TJ, 0>(acc, bias, ep, M, N, tm * BM + wm * 32 * TI,
                                  tn * BN + wn * 32 * TJ, lane);
}

// ------------------------------------------- one wave per SIMD, 256 x 256/192

// 256 x (64 TJ) tile on four waves (2 x 2, each 128 x 32 TJ as 4 x TJ
// accumulators, held in the accumulation registers): one wave per SIMD, so
// the latency is hidden inside each wave rather than by a second wave.  The
// fragments of sub-step ks+1 are read from LDS while the MFMAs of sub-step
// ks run; the global loads run two K steps ahead; and the one barrier of a
// K step sits before its last sub-step's MFMAs, so the next step's first
// fragment reads overlap them.  Needs an even number of K steps and element
// offsets below 2^31.  A launch of more than one round of tiles runs
// persistent (TileMap::persist): one workgroup per CU walks its XCD's share
// of the tiles, taking each next tile's first loads while the last tile's
// output stores drain (MI355X, in-iteration: 175B QKV and FFN1 0.6-2%,
// 13B QKV and FFN1 0.6-0.8% faster; ORCA_GEMM_PERSIST=0 turns it off).
constexpr int W4_THREADS = 256;

// The bf16 epilogue of a 256 x (64 TJ) four-wave tile, staged through LDS
// (the K-step stages, free once the K loop is done).  Each wave writes its
// accumulators plus bias (GeLU applied) as bf16 into a row-major tile whose
// row stride is BN + 4 elements (consecutive rows start 8 bytes apart
// modulo the bank cycle: the writes are conflict-free), then every thread
// stores 16-byte pieces of whole rows: a store instruction covers 1 KB of
// two to three rows, where the accumulator layout gives 32 rows x 16 bytes.
// Same values, same bits as the direct epilogue.  MI355X, in-iteration,
// same box: FFN1 -1.6% (175B layer) and -1.9% (13B), the 175B layer's QKV
// projection -2.4%.
// Measured and not taken: the fp32 residual epilogue staged in two halves
// of 128 rows (175B output projection +1.9% with 8 residual pieces in
// flight per thread, +1.2% with 16, +5% with 32; the 13B output projection
// -1.4%; FFN2 unchanged), and the QKV projection on the 256 x 192 tile,
// whose 24 pieces a row do not divide the workgroup (each piece looking up
// its head block: +1.6%; 192 threads keeping one piece's column each: no
// faster).
// The fp32 partial sums of a split-tail tile into its dense [BM][BN] block,
// staged through LDS in two halves of 128 rows (row stride BN + 4 floats),
// then stored as 16-byte pieces of whole rows: the block is contiguous, so
// a store instruction covers 1 KB.  It also frees the registers the direct
// store spilled.  MI355X, 175B layer in-iteration (three alternations):
// QKV and FFN1 with their tails -0.3%.
template <int TJ>
__device__ __forceinline__ void store_partial_staged(const f32x16_t (&acc)[4][TJ], float* dst,
                                                     int wm, int wn, int lane, int tid,
                                                     uint16_t* smem) {
  constexpr int TI = 4, BN = 64 * TJ, SLD = BN + 4, HM = 128, CPF = BN / 4;
  static_assert(HM * SLD * 4 <= (2 * 256 * LDK + 2 * BN * LDK) * 2, "half a tile fits");
  float* const sF = reinterpret_cast<float*>(smem);
  const int mr = lane & 31, nh = (lane >> 5) * 4, c0 = wn * 32 * TJ;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    __syncthreads();   // the last fragment reads, or the last half's LDS reads, are done
    if (wm == hf) {
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            *reinterpret_cast<float4*>(&sF[(32 * i + mr) * SLD + c0 + 32 * j + 8 * q + nh]) =
                make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                            acc[i][j][4 * q + 3]);
    }
    __syncthreads();
    float* const out = dst + (size_t)hf * HM * BN;
#pragma unroll 4
    for (int idx = tid; idx < HM * CPF; idx += W4_THREADS) {
      const int r = idx / CPF, c = idx - r * CPF;
      *reinterpret_cast<float4*>(out + (size_t)r * BN + 4 * c) =
          *reinterpret_cast<const float4*>(&sF[r * SLD + 4 * c]);
    }
  }
}

template <int EPI, int TJ>
__device__ __forceinline__ void store_tile_staged(const f32x16_t (&acc)[4][TJ],
                                                  const bf16* __restrict__ bias,
                                                  const EpiParams& ep, int M, int N, int tm,
                                                  int tn, int wm, int wn, int lane, int tid,
                                                  uint16_t* smem) {
  constexpr int TI = 4, BM = 256, BN = 64 * TJ, SLD = BN + 4;
  constexpr int CPR = BN / 8;   // 16-byte pieces per row
  static_assert(BM * SLD <= 2 * BM * LDK + 2 * BN * LDK, "the tile fits the stages");
  static_assert(EPI != EPI_QKV || W4_THREADS % CPR == 0, "QKV: a thread keeps its columns");
  const int mr = lane & 31, nh = (lane >> 5) * 4;
  const int c0 = wn * 32 * TJ, r0 = wm * 32 * TI;
  float bq[TJ][4][4];
#pragma unroll
  for (int j = 0; j < TJ; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int n = min(tn * BN + c0 + 32 * j + 8 * q + nh, N - 4);
      const uint2 w = *reinterpret_cast<const uint2*>(bias + n);
      bq[j][q][0] = bf16_lo(w.x);
      bq[j][q][1] = bf16_hi(w.x);
      bq[j][q][2] = bf16_lo(w.y);
      bq[j][q][3] = bf16_hi(w.y);
    }
  __syncthreads();   // every wave's last fragment reads are done
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = acc[i][j][4 * q + e] + bq[j][q][e];
          if constexpr (EPI == ORCA_EPI_BIAS_GELU) v[e] = gelu_tanh(v[e]);
        }
        *reinterpret_cast<uint2*>(&smem[(r0 + 32 * i + mr) * SLD + c0 + 32 * j + 8 * q + nh]) =
            make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      }
  __syncthreads();
  if constexpr (EPI == EPI_QKV) {
    // a thread keeps piece c of rows tid / CPR + 8 k: its destination column
    // (eight columns of one head of Q, K or V) is fixed
    const int c = tid % CPR, n = tn * BN + 8 * c;
    if (n < N) {
      const EpiCol<bf16, EPI> col(ep, n);
#pragma unroll 4
      for (int r = tid / CPR; r < BM && tm * BM + r < M; r += W4_THREADS / CPR) {
        const int m = tm * BM + r;
        const int dst = col.slot ? ep.qkv.row_dst[m] : m;
        *reinterpret_cast<uint4*>(col.ptr + (size_t)dst * col.stride) =
            *reinterpret_cast<const uint4*>(&smem[r * SLD + 8 * c]);
      }
    }
  } else {
    bf16* const out = static_cast<bf16*>(ep.out);
#pragma unroll 4
    for (int idx = tid; idx < BM * CPR; idx += W4_THREADS) {
      const int r = idx / CPR, c = idx - r * CPR;
      const int m = tm * BM + r, n = tn * BN + 8 * c;
      if (m < M && n < N)
        *reinterpret_cast<uint4*>(out + (size_t)m * ep.ldo + n) =
            *reinterpret_cast<const uint4*>(&smem[r * SLD + 8 * c]);
    }
  }
}

template <int EPI, int TJ>
__global__ __launch_bounds__(W4_THREADS, 1)
void gemm_w4_kernel(const bf16* __restrict__ A, const bf16* __restrict__ W,
                    const bf16* __restrict__ bias, EpiParams ep, int M, int N, int K,
                    TileMap map) {
  constexpr int TI = 4, BM = 256, BN = 64 * TJ;
  // 16-byte chunks per lane and K step: LA of A rows, then LB of W rows
  constexpr int LA = BM * 8 / W4_THREADS, LB = BN * 8 / W4_THREADS, NC = LA + LB;
  // the two K-step stages.  The staged epilogues (bf16 outputs and the
  // split tail's partial sums) lay them out in one buffer, which holds the
  // output tile after the K loop; the residual epilogue keeps two arrays
  // (one buffer costs its register allocation more spills; only the
  // variables a form uses are allocated)
  constexpr bool STAGED = EPI == ORCA_EPI_BIAS || EPI == ORCA_EPI_BIAS_GELU ||
                          (EPI == EPI_QKV && TJ == 4) || EPI == EPI_PARTIAL;
  __shared__ __attribute__((aligned(16))) uint16_t smem_w4[2 * BM * LDK + 2 * BN * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t sA_w4[2][BM * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t sB_w4[2][BN * LDK];
  uint16_t (*const sA)[BM * LDK] =
      STAGED ? reinterpret_cast<uint16_t (*)[BM * LDK]>(smem_w4) : sA_w4;
  uint16_t (*const sB)[BN * LDK] =
      STAGED ? reinterpret_cast<uint16_t (*)[BN * LDK]>(smem_w4 + 2 * BM * LDK) : sB_w4;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  // this workgroup's K steps: all of K outside a split tail.  A tail
  // workgroup sets its K range per tile below (KT steps from the byte
  // offset koff into the unshifted operands)
  const int k0 = EPI == EPI_PARTIAL ? 0 : blockIdx.y * map.kt_per_split;
  const int KT_all = min(K / BK - k0, map.kt_per_split);
  A += (size_t)k0 * BK;
  W += (size_t)k0 * BK;

  // loads: lane tid moves chunk tid % 8 of rows tid / 8 + 32 i; byte
  // offsets from a uniform base keep each address to one register
  const int ch = tid & 7;
  uint32_t offA[LA], offB[LB];
  // A rows past M (in the last row tile) read zeros: their offset is the
  // resource's size, and a buffer read at or past num_records returns 0.
  // The clock is power-limited, and MFMAs on zero operands draw less than
  // on copies of a real row (the 13B iteration -1.0%, the 175B-layer one
  // -0.6%).  Near 4 GB of A, where the size plus a K step's offset could
  // wrap 32 bits, the rows are clamped to M - 1 instead.
  const size_t a_bytes = ((size_t)M * K - (size_t)k0 * BK) * 2;
  const bool zero_rows = a_bytes + (size_t)K * 2 < 0xffffffffu;
  const int oL = (tid >> 3) * LDK + ch * 8;   // chunk i lands 32 rows further down
  typedef uint32_t Stage __attribute__((ext_vector_type(4 * NC)));
  typedef uint32_t U4 __attribute__((ext_vector_type(4)));
  Stage s0, s1;
  // buffer loads: a 32-bit lane offset plus the K step's offset in a scalar
  // register, so no 64-bit address is formed per load.  The resource's last
  // word (0x00020000) selects raw 32-bit data, as gfx9-family raw buffer
  // loads expect; num_records is the operand's size (valid rows never reach
  // past it; A's padding rows start at it and read zeros)
  const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
      (void*)A, (short)0,
      (int)(uint32_t)std::min<size_t>(((size_t)M * K - (size_t)k0 * BK) * 2, 0xffffffffu),
      0x00020000);
  const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc(
      (void*)W, (short)0,
      (int)(uint32_t)std::min<size_t>(((size_t)N * K - (size_t)k0 * BK) * 2, 0xffffffffu),
      0x00020000);
// chunk c of a stage: c < LA are A rows, the rest W rows
#define ORCA_W4_LOAD(S, KS, C0, C1)                                                           \
  {                                                                                           \
    const int kb = (KS) * BK * 2 + koff;                                                      \
    _Pragma("unroll") for (int c = (C0); c < (C1); ++c) {                                     \
      const U4 t = c < LA ? __builtin_amdgcn_raw_buffer_load_b128(rA, offA[c], kb, 0)         \
                          : __builtin_amdgcn_raw_buffer_load_b128(rB, offB[c - LA], kb, 0);   \
      S[4 * c] = t.x; S[4 * c + 1] = t.y; S[4 * c + 2] = t.z; S[4 * c + 3] = t.w;             \
    }                                                                                         \
  }
#define ORCA_W4_STORE(S, BUF, C0, C1)                                                         \
  {                                                                                           \
    _Pragma("unroll") for (int c = (C0); c < (C1); ++c)                                       \
        *reinterpret_cast<uint4*>(c < LA ? &sA[BUF][oL + c * 32 * LDK]                        \
                                         : &sB[BUF][oL + (c - LA) * 32 * LDK]) =              \
            make_uint4(S[4 * c], S[4 * c + 1], S[4 * c + 2], S[4 * c + 3]);                   \
  }

  const int fr = lane & 31, fk = (lane >> 5) * 8;
  const int a_off = (wm * 32 * TI + fr) * LDK + fk, b_off = (wn * 32 * TJ + fr) * LDK + fk;
  f32x16_t acc[TI][TJ];
  bf16x8_t fa0[TI], fb0[TJ], fa1[TI], fb1[TJ];
#define ORCA_W4_FRAGS(FA, FB, BUF, KS)                                                        \
  _Pragma("unroll") for (int i = 0; i < TI; ++i) FA[i] =                                      \
      *reinterpret_cast<const bf16x8_t*>(&sA[BUF][a_off + i * 32 * LDK + (KS) * 16]);         \
  _Pragma("unroll") for (int j = 0; j < TJ; ++j) FB[j] =                                      \
      *reinterpret_cast<const bf16x8_t*>(&sB[BUF][b_off + j * 32 * LDK + (KS) * 16]);
  // W as the first operand: each accumulator holds C^T (see store_wave_tile_t)
#define ORCA_W4_MFMA(FA, FB)                                                                  \
  _Pragma("unroll") for (int i = 0; i < TI; ++i)                                              \
      _Pragma("unroll") for (int j = 0; j < TJ; ++j) acc[i][j] =                              \
          __builtin_amdgcn_mfma_f32_32x32x16_bf16(FB[j], FA[i], acc[i][j], 0, 0, 0);
  // step kt (LDS buffer CUR): loads of step kt+2 into LS, step kt+1 from SS
  // into the other buffer, then the four sub-steps with the barrier before
  // the last one's MFMAs
  // sched_group_barrier masks: MFMA 0x8, VMEM read 0x20, DS read 0x100,
  // DS write 0x200.  A K step is four phases of NM = 4 TJ MFMAs (one
  // sub-step each), fenced by scheduling barriers.  The step's NC global
  // loads (of step kt+2), NC LDS writes (of step kt+1, into the other
  // buffer) and the fragment reads are spread evenly over them, so neither
  // the LDS nor the address path sees a burst: each phase reads the next
  // sub-step's fragments and issues a quarter of the loads; phases a-c
  // write a third of the chunks each.  The barrier sits between phases c
  // and d: phase d's fragment reads are of the next K step's first sub-step.
  constexpr int NM = TI * TJ, NR = TI + TJ;
  constexpr int G1 = NC / 4, G2 = NC / 2, G3 = 3 * NC / 4, W1 = NC / 3, W2 = 2 * NC / 3;
#define ORCA_W4_SPREAD(NG, NW)                                                                \
  _Pragma("unroll") for (int j = 0; j < NM; ++j) {                                            \
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                        \
    if (j < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                            \
    if (((j + 1) * (NG)) / NM > (j * (NG)) / NM)                                              \
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);                                      \
    if (((j + 1) * (NW)) / NM > (j * (NW)) / NM)                                              \
      __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);                                      \
  }
#define ORCA_W4_STEP(CUR, LS, SS)                                                             \
  {                                                                                           \
    const int kl = min(kt + (CUR) + 2, KT - 1);                                               \
    ORCA_W4_FRAGS(fa1, fb1, CUR, 1)                                                           \
    ORCA_W4_LOAD(LS, kl, 0, G1)                                                               \
    ORCA_W4_STORE(SS, (CUR) ^ 1, 0, W1)                                                       \
    ORCA_W4_MFMA(fa0, fb0)                                                                    \
    ORCA_W4_SPREAD(G1, W1)                                                                    \
    __builtin_amdgcn_sched_barrier(0);                                                        \
    ORCA_W4_FRAGS(fa0, fb0, CUR, 2)                                                           \
    ORCA_W4_LOAD(LS, kl, G1, G2)                                                              \
    ORCA_W4_STORE(SS, (CUR) ^ 1, W1, W2)                                                      \
    ORCA_W4_MFMA(fa1, fb1)                                                                    \
    ORCA_W4_SPREAD(G2 - G1, W2 - W1)                                                          \
    __builtin_amdgcn_sched_barrier(0);                                                        \
    ORCA_W4_FRAGS(fa1, fb1, CUR, 3)                                                           \
    ORCA_W4_LOAD(LS, kl, G2, G3)                                                              \
    ORCA_W4_STORE(SS, (CUR) ^ 1, W2, NC)                                                      \
    ORCA_W4_MFMA(fa0, fb0)                                                                    \
    ORCA_W4_SPREAD(G3 - G2, NC - W2)                                                          \
    __builtin_amdgcn_sched_barrier(0);                                                        \
    __syncthreads();                                                                          \
    ORCA_W4_FRAGS(fa0, fb0, (CUR) ^ 1, 0)                                                     \
    ORCA_W4_LOAD(LS, kl, G3, NC)                                                              \
    ORCA_W4_MFMA(fa1, fb1)                                                                    \
    ORCA_W4_SPREAD(NC - G3, 0)                                                                \
    __builtin_amdgcn_sched_barrier(0);                                                        \
  }
  // this workgroup's tiles: one (local = its launch index through the XCD
  // remap), or in a persistent launch the tiles lo + i, lo + i + G / 8, ...
  // of its XCD's contiguous share [lo, hi), i = blockIdx.x / 8, G / 8
  // workgroups per XCD, so the XCD's workgroups take consecutive tiles at
  // every turn, as the rounds of a one-tile launch do
  int t_first, t_stride, t_count;
  if (map.persist > 0) {
    const int x = blockIdx.x % 8, per = gridDim.x / 8;
    const int q = map.persist / 8, r = map.persist % 8;
    const int lo = x * q + min(x, r), hi = lo + q + (x < r ? 1 : 0);
    t_first = lo + blockIdx.x / 8;
    t_stride = per;
    t_count = t_first < hi ? (hi - t_first + per - 1) / per : 0;
  } else {
    t_first = xcd_remap(blockIdx.x, gridDim.x);
    t_stride = 1;
    t_count = EPI == EPI_PARTIAL && map.sk_kt > 0 ? sk_segments(map, t_first) : 1;
  }
  for (int it = 0; it < t_count; ++it) {
    int local = t_first + it * t_stride, KT = KT_all, koff = 0;
    size_t slot = 0;   // a tail tile's fp32 partial tile
    if constexpr (EPI == EPI_PARTIAL) {
      if (map.sk_kt > 0) {
        int kfirst;
        sk_segment(map, t_first, it, local, kfirst, KT, slot);
        koff = kfirst * BK * 2;
      } else {
        const int kfirst = blockIdx.y * map.kt_per_split;
        KT = min(K / BK - kfirst, map.kt_per_split);
        koff = kfirst * BK * 2;
        slot = (size_t)blockIdx.y * map.n_tail + local;
      }
    }
    int tm, tn;
    tile_of(map.tile_base + local, map.tiles_m, map.ntiles, map.group, tm, tn);
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int row = tm * BM + (tid >> 3) + 32 * i;
      offA[i] = row < M ? (uint32_t)(row * K + ch * 8) * 2u
                        : zero_rows ? (uint32_t)a_bytes : (uint32_t)((M - 1) * K + ch * 8) * 2u;
    }
#pragma unroll
    for (int i = 0; i < LB; ++i)
      offB[i] = (uint32_t)(min(tn * BN + (tid >> 3) + 32 * i, N - 1) * K + ch * 8) * 2u;
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    ORCA_W4_LOAD(s0, 0, 0, NC)
    ORCA_W4_LOAD(s1, min(1, KT - 1), 0, NC)
    // the previous tile's last fragment reads of buffer 0 are done
    if (it > 0) __syncthreads();
    ORCA_W4_STORE(s0, 0, 0, NC)
    __syncthreads();
    ORCA_W4_FRAGS(fa0, fb0, 0, 0)
    for (int kt = 0; kt < KT; kt += 2) {
      ORCA_W4_STEP(0, s0, s1)
      ORCA_W4_STEP(1, s1, s0)
    }
#undef ORCA_W4_STEP
#undef ORCA_W4_SPREAD
#undef ORCA_W4_MFMA
#undef ORCA_W4_FRAGS
#undef ORCA_W4_LOAD
#undef ORCA_W4_STORE
    if constexpr (EPI == EPI_PARTIAL) {
      // split tail: this workgroup's sums of the tile into its partial tile
      // (split-major for an even split; main, then helper, parts)
      store_partial_staged<TJ>(acc, static_cast<float*>(ep.out) + slot * BM * BN, wm, wn, lane,
                               tid, smem_w4);
    } else if constexpr (STAGED) {
      store_tile_staged<EPI, TJ>(acc, bias, ep, M, N, tm, tn, wm, wn, lane, tid, smem_w4);
    } else {
      store_wave_tile_t<EPI, TI, TJ>(acc, bias, ep, M, N, tm * BM + wm * 32 * TI,
                                     tn * BN + wn * 32 * TJ, lane);
    }
  }
}

// The split-K tail of a hybrid four-wave launch: adds the partial sums of
// each tail tile in K order, then the bias and the epilogue, four
// consecutive columns per thread (they lie in one head of one block for the
// QKV projection, as the head dim is a multiple of four).  An even split
// leaves `splits` partial tiles per tail tile, split-major (tile t's at t,
// t + n_tail, ...); a main-and-helper tail two (t, n_tail + t).
template <int EPI, int BN>
__global__ __launch_bounds__(256) void tail_reduce_kernel(const float* __restrict__ part,
                                                          int splits, TileMap map,
                                                          const bf16* __restrict__ bias,
                                                          EpiParams ep, int M, int N) {
  constexpr int BM = 256, Q = BN / 4;
  const int t = blockIdx.x;
  int tm, tn;
  tile_of(map.tile_base + t, map.tiles_m, map.ntiles, map.group, tm, tn);
  const int count = map.sk_kt > 0 ? 2 : splits;
  const size_t plane = (size_t)map.n_tail * BM * BN;
  for (int idx = blockIdx.y * 256 + threadIdx.x; idx < BM * Q; idx += gridDim.y * 256) {
    const int r = idx / Q, c = (idx - r * Q) * 4;
    const int m = tm * BM + r, n = tn * BN + c;
    if (m >= M || n >= N) continue;
    const float* p = part + (size_t)t * BM * BN + (size_t)r * BN + c;
    float4 v = *reinterpret_cast<const float4*>(p);
    for (int sp = 1; sp < count; ++sp) {
      const float4 u = *reinterpret_cast<const float4*>(p + sp * plane);
      v.x += u.x; v.y += u.y; v.z += u.z; v.w += u.w;
    }
    const uint2 bw = *reinterpret_cast<const uint2*>(bias + n);
    float o[4] = {v.x + bf16_lo(bw.x), v.y + bf16_hi(bw.x), v.z + bf16_lo(bw.y),
                  v.w + bf16_hi(bw.y)};
    if constexpr (EPI == ORCA_EPI_BIAS_RESID) {
      float4* q = reinterpret_cast<float4*>(static_cast<float*>(ep.out) + (size_t)m * ep.ldo + n);
      const float4 old = *q;
      *q = make_float4(old.x + o[0], old.y + o[1], old.z + o[2], old.w + o[3]);
    } else {
      if constexpr (EPI == ORCA_EPI_BIAS_GELU) {
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = gelu_tanh(o[e]);
      }
      const EpiCol<bf16, EPI> col(ep, n);
      const int slot = EPI == EPI_QKV ? ep.qkv.row_dst[m] : 0;
      *reinterpret_cast<uint2*>(col.ptr + (size_t)(col.slot ? slot : m) * col.stride) =
          make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
    }
  }
}

// --------------------------------- one wave per SIMD, operands DMA'd to LDS

// The same 256 x (64 TJ) tile on four waves, with the operands moved from
// HBM straight into LDS by the buffer loads' LDS mode (gfx950 moves 16
// bytes per lane this way): no staging registers, no LDS write
// instructions.  K step 32, four LDS stages, so the loads of step kt+4 are
// issued three steps before they are read.  A load writes lane l's 16 bytes
// at (M0 + 16 l), so the LDS layout follows the lane order: 64-byte rows
// (32 bf16 of one K step) with the four 16-byte chunks of row r permuted by
// XOR with swz(r) = ((r >> 1) ^ (r >> 3)) & 3, which spreads the eight (or
// sixteen) rows one ds_read_b128 serves over distinct LDS banks; each lane
// loads the global chunk that belongs at its LDS slot.
typedef uint32_t rsrc_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ rsrc_t buffer_rsrc(const void* base, size_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  rsrc_t r;
  r.x = (uint32_t)p;
  r.y = (uint32_t)(p >> 32) & 0xffffu;   // stride 0
  r.z = (uint32_t)std::min<size_t>(bytes, 0xffffffffu);
  r.w = 0x00020000u;                     // raw 32-bit data (gfx9 family)
  return r;
}

__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// One 16-byte-per-lane buffer load into LDS at lds + 16 * lane.  Written as
// assembly so that the compiler does not count it among the LDS writes it
// orders: with the builtin it waits for every load in flight before each LDS
// read, which serialises the stages.  The caller waits (vmcnt) and meets the
// workgroup barrier before reading what it wrote.  M0 is restored.
__device__ __forceinline__ void dma_b128(const rsrc_t& r, uint32_t lds, uint32_t voff,
                                         uint32_t soff) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(voff), "s"(r), "s"(soff)
      : "memory");
}

// s_waitcnt for the vector-memory counter only
#define ORCA_WAIT_VMCNT(N) \
  __builtin_amdgcn_s_waitcnt(((N) & 0xf) | (((N) >> 4) << 14) | (0x7 << 4) | (0xf << 8))

template <int EPI, int TJ, int DK>
__global__ __launch_bounds__(W4_THREADS, 1)
void gemm_d4_kernel(const bf16* __restrict__ A, const bf16* __restrict__ W,
                    const bf16* __restrict__ bias, EpiParams ep, int M, int N, int K,
                    int tiles_m, int group_m) {
  constexpr int TI = 4, BM = 256, BN = 64 * TJ;
  constexpr int ROWB = DK * 2;                    // bytes per row and K step
  constexpr int CPR = ROWB / 16;                  // 16-byte chunks per row
  constexpr int RPI = 1024 / ROWB;                // rows one 1 KB load fills
  constexpr int NS = DK == 32 ? 4 : 2;            // LDS stages
  constexpr int NSUB = DK / 16;                   // MFMA sub-steps per K step
  constexpr int STAGE = (BM + BN) * ROWB;         // bytes per stage
  constexpr int NIW = (BM + BN) / (4 * RPI);      // 1 KB loads per wave and stage
  constexpr int NM = TI * TJ, NR = TI + TJ;
  static_assert(DK == 32 || DK == 64, "K step");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NS * STAGE];

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  int tm, tn;
  tile_of(logical, tiles_m, gridDim.x, group_m, tm, tn);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int KT = K / DK;
  // chunk permutation of LDS row r (a function of r mod 32): the rows one
  // ds_read_b128 serves land in distinct banks for 8 and for 16 lanes
  auto swz = [](int r) {
    return DK == 32 ? ((r >> 1) ^ (r >> 3)) & 3 : (r ^ ((r >> 3) & 3)) & 7;
  };

  const rsrc_t rA = buffer_rsrc(A, (size_t)M * K * 2);
  const rsrc_t rB = buffer_rsrc(W, (size_t)N * K * 2);
  // load j of this wave fills stage rows RPI c .. RPI c + RPI-1, c = 4 j +
  // wave (rows 0 .. BM-1 hold A, the rest W); lane l takes row RPI c +
  // l / CPR and LDS chunk l % CPR, which holds the row's global chunk
  // (l % CPR) ^ swz(row)
  uint32_t voff[NIW];
#pragma unroll
  for (int j = 0; j < NIW; ++j) {
    const int r = RPI * (4 * j + wave) + lane / CPR;
    const int c = (lane % CPR) ^ swz(r);
    const int g = j < BM / (4 * RPI) ? min(tm * BM + r, M - 1) : min(tn * BN + r - BM, N - 1);
    voff[j] = (uint32_t)g * (uint32_t)K * 2u + (uint32_t)c * 16u;
  }
  const uint32_t lds0 = lds_address(smem) + (uint32_t)wave * 1024u;
#define ORCA_D4_LOAD(J, ST, KS)                                                               \
  dma_b128((J) < BM / (4 * RPI) ? rA : rB, lds0 + (ST) * STAGE + (J) * 4096, voff[J],         \
           (KS) * ROWB)

  // fragment reads: lane row fr, sub-step ks takes logical chunk 2 ks + h
  const int fr = lane & 31, h = lane >> 5, sw = swz(fr);
  int ro[NSUB];
#pragma unroll
  for (int ks = 0; ks < NSUB; ++ks) ro[ks] = fr * ROWB + ((2 * ks + h) ^ sw) * 16;
  const uint8_t* fa_base = smem + (wm * 32 * TI) * ROWB;
  const uint8_t* fb_base = smem + (BM + wn * 32 * TJ) * ROWB;
#define ORCA_D4_FRAG(U, FA, FB, ST, RO)                                                       \
  if ((U) < TI)                                                                              \
    FA[(U) < TI ? (U) : 0] = *reinterpret_cast<const bf16x8_t*>(                              \
        fa_base + (ST) * STAGE + (U) * 32 * ROWB + (RO));                                     \
  else if ((U) < NR)                                                                         \
    FB[(U) < NR && (U) >= TI ? (U) - TI : 0] = *reinterpret_cast<const bf16x8_t*>(            \
        fb_base + (ST) * STAGE + ((U) - TI) * 32 * ROWB + (RO));
#define ORCA_D4_MFMA(U, FA, FB)                                                               \
  acc[(U) / TJ][(U) % TJ] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(                          \
      FB[(U) % TJ], FA[(U) / TJ], acc[(U) / TJ][(U) % TJ], 0, 0, 0);

  f32x16_t acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  bf16x8_t fa0[TI], fb0[TJ], fa1[TI], fb1[TJ];

#pragma unroll
  for (int st = 0; st < NS; ++st)
#pragma unroll
    for (int j = 0; j < NIW; ++j) ORCA_D4_LOAD(j, st, min(st, KT - 1));
  ORCA_WAIT_VMCNT((NS - 1) * NIW);
  __syncthreads();
#pragma unroll
  for (int u = 0; u < NR; ++u) { ORCA_D4_FRAG(u, fa0, fb0, 0, ro[0]) }

  for (int kt = 0; kt < KT; ++kt) {
    const int st = kt % NS, nst = (kt + 1) % NS;
    // sub-steps 0 .. NSUB-2: each one's MFMAs with the next one's fragment
    // reads (two register sets, alternating)
#pragma unroll
    for (int ks = 0; ks + 1 < NSUB; ++ks) {
#pragma unroll
      for (int u = 0; u < NM; ++u) {
        if (ks % 2 == 0) {
          ORCA_D4_FRAG(u, fa1, fb1, st, ro[ks + 1])
          ORCA_D4_MFMA(u, fa0, fb0)
        } else {
          ORCA_D4_FRAG(u, fa0, fb0, st, ro[ks + 1])
          ORCA_D4_MFMA(u, fa1, fb1)
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // this wave's loads of step kt+1 have landed (later steps may still be
    // in flight); after the barrier every wave's have, and no wave reads
    // stage st any more
    ORCA_WAIT_VMCNT((NS - 2) * NIW);
    __syncthreads();
    // the last sub-step's MFMAs, with the loads of step kt+NS into stage st
    // and the reads of the next step's first fragments
#pragma unroll
    for (int u = 0; u < NM; ++u) {
#pragma unroll
      for (int j = u * NIW / NM; j < (u + 1) * NIW / NM; ++j)
        ORCA_D4_LOAD(j, st, min(kt + NS, KT - 1));
      ORCA_D4_FRAG(u, fa0, fb0, nst, ro[0])
      ORCA_D4_MFMA(u, fa1, fb1)
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  ORCA_WAIT_VMCNT(0);
#undef ORCA_D4_MFMA
#undef ORCA_D4_FRAG
#undef ORCA_D4_LOAD
  store_wave_tile_t<EPI, TI, TJ>(acc, bias, ep, M, N, tm * BM + wm * 32 * TI,
                                 tn * BN + wn * 32 * TJ, lane);
}

// ---------------------------------------------------------------- few rows

// Few rows (iterations made mostly of increment rows) make the Linear
// layers weight-streaming: every weight is read once per iteration and the
// MFMA units idle, while 256 x 256 or 128 x 128 tiles would leave most CUs
// without work (a 5120-column layer at 64 rows has 40 of them).  The
// split-K path runs the kernel above on 32 x 128, 64 x 128 or 128 x 128
// tiles with grid.y splitting K (EPI_PARTIAL: fp32 partial sums to
// [splits][M][N], no bias), so the grid holds enough workgroups to keep HBM
// busy with the same coalesced 128-byte row loads; this kernel then adds
// the splits, the bias and the epilogue, four columns per thread.
template <int EPI>
__global__ __launch_bounds__(256) void skinny_reduce_kernel(const float* __restrict__ part,
                                                            int splits,
                                                            const bf16* __restrict__ bias,
                                                            EpiParams ep, int M, int N) {
  using OutT = typename std::conditional<EPI == ORCA_EPI_BIAS_RESID, float, bf16>::type;
  const int n4 = N / 4;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= M * n4) return;
  const int m = idx / n4, n = (idx - m * n4) * 4;
  const size_t stride = (size_t)M * N, base = (size_t)m * N + n;
  float bb[4];   // the bias read before the first write
#pragma unroll
  for (int c = 0; c < 4; ++c) bb[c] = load_f32(bias + n + c);
  const int dst = EPI == EPI_QKV ? ep.qkv.row_dst[m] : 0;
  float4 old = make_float4(0.f, 0.f, 0.f, 0.f);   // the residual, read up front
  if constexpr (EPI == ORCA_EPI_BIAS_RESID)
    old = *reinterpret_cast<const float4*>(static_cast<const float*>(ep.out) +
                                           (size_t)m * ep.ldo + n);
  // the planes are read four at a time, all four issued before any is
  // added (a clamped index re-reads the last plane and is not added): one
  // load per loop trip made every plane a separate round trip
  float4 v = *reinterpret_cast<const float4*>(part + base);
  for (int s0 = 1; s0 < splits; s0 += 4) {
    float4 t[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      t[u] = *reinterpret_cast<const float4*>(part + min(s0 + u, splits - 1) * stride + base);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      // a select, not a branch: behind a branch the load sinks into it
      const bool on = s0 + u < splits;
      v.x += on ? t[u].x : 0.f; v.y += on ? t[u].y : 0.f;
      v.z += on ? t[u].z : 0.f; v.w += on ? t[u].w : 0.f;
    }
  }
  if constexpr (EPI == ORCA_EPI_BIAS_RESID) {
    *reinterpret_cast<float4*>(static_cast<float*>(ep.out) + (size_t)m * ep.ldo + n) =
        make_float4(old.x + (v.x + bb[0]), old.y + (v.y + bb[1]), old.z + (v.z + bb[2]),
                    old.w + (v.w + bb[3]));
    return;
  }
  const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const EpiCol<OutT, EPI> col(ep, n + c);
    col.store(m, dst, vv[c] + bb[c]);
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
    const EpiCol<float, EPI> col(ep, n);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = tm * 64 + ty * 4 + i;
      if (m < M) col.store(m, EPI == EPI_QKV ? ep.qkv.row_dst[m] : 0, acc[i][j] + bias[n]);
    }
  }
}

// ---------------------------------------------------------------- launcher

// Tile variants (wave grid x per-wave 32x32 tiles):
//   0: 2x2 waves, 2x2 tiles -> 128 x 128, 256 threads, 2 workgroups / CU
//   3: 4x2 waves, 2x4 tiles -> 256 x 256, 512 threads
//   6: as 3, with two K steps of global loads in flight
//   7: as 0, with two K steps of global loads in flight
//   8: 4x2 waves, 2x3 tiles -> 256 x 192, 512 threads, two K steps in flight
//  10: split-K (see plan_gemm)
//  11: wave-specialised 256 x 256 (eight MFMA waves, four loader waves)
//  12: four waves, 4x4 tiles each -> 256 x 256, one wave per SIMD
//  13: four waves, 4x3 tiles each -> 256 x 192, one wave per SIMD
// (6, 7 and 8 need an even number of K steps and fall back to 3, 0 and the
// one-step 256 x 192 form; 11, 12 and 13 need an even number of K steps and
// element offsets below 2^31 and fall back to 6, 6 and 8.  The planner
// picks among 12, 13, 7 and 10; the others stay for tests and sweeps.)
template <int EPI, int WGM, int WGN, int TI, int TJ, bool PIPE = false, bool STREAM_W = false>
static void launch_mfma(const void* a, const void* w, const void* bias, const EpiParams& ep, int m,
                        int n, int k, hipStream_t s, int splits = 1, int kt_per_split = 0) {
  using C = TileCfg<WGM, WGN, TI, TJ>;
  const int tiles_m = (m + C::BM - 1) / C::BM, tiles_n = (n + C::BN - 1) / C::BN;
  hipLaunchKernelGGL((gemm_bf16_kernel<EPI, WGM, WGN, TI, TJ, PIPE, STREAM_W>),
                     dim3(tiles_m * tiles_n, splits), dim3(C::NT), 0, s, (const bf16*)a,
                     (const bf16*)w, (const bf16*)bias, ep, m, n, k, tiles_m,
                     kt_per_split > 0 ? kt_per_split : k / BK);
}

// Split-K plan: tile, tile count, K steps per split, splits.  grid.y splits
// the K steps, an even count per split (the two-step pipeline); each split
// writes fp32 partial sums that skinny_reduce_kernel adds up.
struct SplitPlan {
  int tile;   // 0: 32 x 128, 1: 64 x 128, 2: 128 x 128, 3: 256 x 256
  int tiles, kt_per_split, splits;
};
constexpr int NUM_CU = 256;              // MI355X
constexpr int LDS_PER_CU = 160 * 1024;
static int env_int(const char* name, int dflt) {
  const char* f = getenv(name);
  return f ? atoi(f) : dflt;
}
static void set_splits(int kt, int splits, SplitPlan& p) {
  int per = (kt + splits - 1) / splits;
  if (kt % 2 == 0) per += per & 1;
  p.kt_per_split = per;
  p.splits = (kt + per - 1) / per;
}
static long ceil_div_l(long a, long b) { return (a + b - 1) / b; }

// Launches whose 32/64/128-row tiles are too few to fill the GPU (few rows,
// or at 1,000-2,000 rows a narrow output such as a 1024-wide projection,
// where 128 x 128 tiles leave most CUs idle): split K.  A CU streams about
// as fast with one of these workgroups as with two (and at more rows two
// share its MFMAs), so the time goes as the rounds of NUM_CU workgroups
// times the K steps of one split; the split count minimises
// that, ties going to fewer splits (each split writes and re-reads an fp32
// partial plane), within one round of resident workgroups (two per CU,
// bounded by LDS).  At 64 rows of the 13B layer this gives 2 splits for
// QKV, 6 for the output projection and FFN2, 3 for FFN1 (measured: 2 and
// 6 beat the 4-12 splits that fill 512 slots by 8-15%; 3 beats 2 and 4).
static bool few_rows_plan(int m, int n, int k, SplitPlan& p) {
  if (m > env_int("ORCA_SPLIT_MAX_M", INT_MAX)) return false;   // a cap for sweeps only
  const int kt = k / BK;
  p.tile = m <= 32 ? 0 : m <= 64 ? 1 : 2;
  const int bm = p.tile == 0 ? 32 : p.tile == 1 ? 64 : 128;
  p.tiles = ((m + bm - 1) / bm) * ((n + 127) / 128);
  const int lds = 2 * (bm + 128) * LDK * 2;
  const int resident = NUM_CU * std::max(1, std::min(2, LDS_PER_CU / lds));
  const int target = std::max(1, env_int("ORCA_SPLIT_TARGET", resident));
  if (2 * p.tiles > target) return false;   // enough tiles already
  SplitPlan best = p;
  best.splits = 1;
  best.kt_per_split = kt;
  long best_cost = ceil_div_l(p.tiles, NUM_CU) * (long)kt;
  for (int sp = 2; sp <= std::min(SPLIT_MAX_SPLITS, std::max(1, kt / 4)); ++sp) {
    SplitPlan q = p;
    set_splits(kt, sp, q);
    if ((long)p.tiles * q.splits > target) break;
    const long cost = ceil_div_l((long)p.tiles * q.splits, NUM_CU) * q.kt_per_split;
    if (cost < best_cost) {
      best = q;
      best_cost = cost;
    }
  }
  p = best;
  return p.splits > 1;
}

// Estimated time of the tiled launches, in units of one 256 x 256 tile-round
// per unit of K: rounds of resident workgroups times the output area a CU
// covers per round, over the tile's measured rate relative to the 256 x 256
// four-wave kernel (MI355X, 13B and 175B layer shapes: its 256 x 192 form
// at 0.92, the 128 x 128 eight-wave tile at 0.76).  The last round counts
// whole: a launch that leaves CUs idle in it pays for them.
static double cost_tiled(int v, int m, int n) {
  switch (v) {
    case 12: return ceil_div_l(ceil_div_l(m, 256) * ceil_div_l(n, 256), NUM_CU) * 65536.0;
    case 13: return ceil_div_l(ceil_div_l(m, 256) * ceil_div_l(n, 192), NUM_CU) * 49152.0 / 0.92;
    default: return ceil_div_l(ceil_div_l(m, 128) * ceil_div_l(n, 128), 2 * NUM_CU) * 32768.0 / 0.76;
  }
}
// The tiled variant of least estimated cost; another tile than 256 x 256
// only on a predicted gain of 3% or more (the model is coarse).  Measured
// on the eight 13B and 175B layer shapes, it picks the faster of the two
// four-wave forms on every one.
static int best_tiled(int m, int n, double& best) {
  int v = 12;
  best = cost_tiled(12, m, n) * 0.97;
  for (int c : {13, 7}) {
    const double e = cost_tiled(c, m, n);
    if (e < best) {
      best = e;
      v = c;
    }
  }
  return v;
}

// 256 x 256 tiles with K split by 2-4 (each split at least 40 K steps; its
// partial sums are written and read back once, charged at 15%).
static double cost_big_split(int m, int n, int k, SplitPlan& p) {
  const int kt = k / BK;
  double best = 1e300;
  p.tile = 3;
  p.tiles = (int)(ceil_div_l(m, 256) * ceil_div_l(n, 256));
  // no split unless a candidate below fills the plan
  p.splits = 1;
  p.kt_per_split = kt;
  if (kt % 2) return best;
  for (int sp = 2; sp <= 4 && kt / sp >= 40; ++sp) {
    // the split GEMM runs on the eight-wave 256 x 256 tile (~0.9 of the
    // four-wave rate), and its partial sums cost ~15% more
    const double c = ceil_div_l((long)p.tiles * sp, NUM_CU) * 65536.0 / sp * 1.15 / 0.9;
    if (c < best) {
      best = c;
      set_splits(kt, sp, p);
    }
  }
  return best;
}

// Row-tile group of the four-wave launches (tile_of): groups of 8 when the
// launch has at least 12 row tiles (MI355X, 175B layer shapes at 3,698
// rows: 1-3% faster than row tiles fastest; at 13B's 9 row tiles it made no
// difference).  ORCA_GEMM_GROUP overrides it for sweeps.
static int raster_group(int tiles_m) {
  return env_int("ORCA_GEMM_GROUP", tiles_m >= 12 ? 8 : 0);
}

// Hybrid four-wave launch: the tiles of every full round run as usual, and
// the last round's n_tail tiles run split over K so that the round keeps
// every CU busy; their fp32 partial sums are added by tail_reduce_kernel,
// which applies the epilogue.  ORCA_GEMM_TAIL=0 turns it off.
// * When that round is at most half full: K split by 2-4 (each split an
//   even number of at least 16 K steps), so the round ends in a fraction of
//   a tile's time.  On the 175B layer shape at 3,698 rows: QKV 2,160 tiles
//   = 8 rounds + 112 tiles (2 splits), FFN1 2,880 = 11 rounds + 64 (4).
// * Fuller: the main-and-helper split (sk_segment) on one workgroup per CU,
//   NUM_CU - n_tail of them helpers taking c = ceil(n_tail / helpers) tile
//   remainders each; x balances a main's x steps against a helper's
//   c (kt - x), plus 4 steps for each further segment's loads and partial
//   store.  Taken where the round shrinks by ORCA_GEMM_SK_MIN (64) K steps
//   or more.  On the 175B layer: FFN2 (720 tiles = 2 rounds + 208, 768 steps
//   a tile: 48 helpers, c = 5, x = 644), not the output projection (192
//   steps, x = 160: 32 steps saved).
struct TailPlan {
  int n_dp, n_tail, splits, per;
  int sk_kt;     // main-and-helper: K steps per tile (0: an even split)
  int wgs;       // tail workgroups
  size_t slots;  // fp32 partial tiles in the workspace
};
static bool tail_plan(int tiles, int kt, TailPlan& t) {
  if (!env_int("ORCA_GEMM_TAIL", 1)) return false;
  const int rem = tiles % NUM_CU;
  if (tiles < NUM_CU || rem == 0 || kt % 2) return false;
  t.n_tail = rem;
  t.n_dp = tiles - rem;
  t.sk_kt = 0;
  if (rem > NUM_CU / 2) {
    const int helpers = NUM_CU - rem, c = (rem + helpers - 1) / helpers;
    int best_x = 0, best = kt;
    for (int x = 2; x <= kt - 2; x += 2) {   // even: a segment runs its K steps in pairs
      const int span = std::max(x, c * (kt - x) + 4 * (c - 1));
      if (span <= best) {
        best = span;
        best_x = x;
      }
    }
    if (best_x == 0 || kt - best < env_int("ORCA_GEMM_SK_MIN", 64)) return false;
    t.per = best_x;
    t.sk_kt = kt;
    t.wgs = NUM_CU;
    t.splits = 2;
    t.slots = 2 * (size_t)rem;
    return true;
  }
  int sp = std::min(4, NUM_CU / rem);
  while (sp > 1 && kt / sp < 16) --sp;
  if (sp < 2) return false;
  int per = (kt + sp - 1) / sp;
  per += per & 1;
  t.splits = (kt + per - 1) / per;
  t.per = per;
  t.wgs = rem;
  t.slots = (size_t)rem * t.splits;
  return t.splits >= 2;
}
// the four-wave forms' tile count (bn: 256 or 192)
static int w4_tiles(int m, int n, int bn) { return ((m + 255) / 256) * ((n + bn - 1) / bn); }
static bool w4_ok(int m, int n, int k) {
  return k >= 2 * BK && (k / BK) % 2 == 0 && (long)std::max(m, n) * k < (1L << 31);
}

// The launch for one bf16 problem: a tiled variant, or split-K (`split`
// filled, variant 10).  ORCA_GEMM_VARIANT=<n> pins the variant.
static int plan_gemm(int m, int n, int k, SplitPlan& split) {
  int pinned = -1;
  if (const char* f = getenv("ORCA_GEMM_VARIANT")) {
    const int v = atoi(f);
    if (v == 0 || v == 3 || v == 6 || v == 7 || v == 8 || (v >= 10 && v <= 15)) pinned = v;
  }
  if (pinned >= 0 && pinned != 10) return pinned;
  if (m >= 1 && k % BK == 0 && n % 4 == 0) {
    if (few_rows_plan(m, n, k, split)) return 10;
    double best;
    const int v = best_tiled(m, n, best);
    SplitPlan bs{};
    if (cost_big_split(m, n, k, bs) < best || pinned == 10) {
      if (bs.splits > 1 && bs.splits <= SPLIT_MAX_SPLITS) {
        split = bs;
        return 10;
      }
    }
    return v;
  }
  return 7;
}

int linear_plan_variant(int dtype, int m, int n, int k) {
  if (dtype != ORCA_BF16) return -1;   // the fp32 FMA kernel
  SplitPlan sp{};
  const int v = plan_gemm(m, n, k, sp);
  const bool even = (k / BK) % 2 == 0;
  switch (v) {
    case 11: return even && (long)std::max(m, n) * k < (1L << 31) ? 11 : (even ? 6 : 3);
    case 12: return even && k >= 2 * BK && (long)std::max(m, n) * k < (1L << 31) ? 12 : (even ? 6 : 3);
    case 13: return even && k >= 2 * BK && (long)std::max(m, n) * k < (1L << 31) ? 13 : 8;
    case 14: return (long)std::max(m, n) * k < (1L << 31) ? 14 : (even ? 6 : 3);
    case 15: return (long)std::max(m, n) * k < (1L << 31) ? 15 : 8;
    default: return v;
  }
}

size_t linear_workspace_bytes(int dtype, int m, int n, int k) {
  SplitPlan p{};
  if (dtype != ORCA_BF16 || m < 1) return 0;
  const int v = plan_gemm(m, n, k, p);
  if (v == 10) return (size_t)p.splits * m * n * sizeof(float);
  if ((v == 12 || v == 13) && w4_ok(m, n, k)) {
    const int bn = v == 12 ? 256 : 192;
    TailPlan t;
    if (tail_plan(w4_tiles(m, n, bn), k / BK, t)) return t.slots * 256 * bn * sizeof(float);
  }
  return 0;
}

template <int WGM, int WGN, int TI, int TJ, bool STREAM_W = false>
static void launch_partial(const SplitPlan& p, const void* a, const void* w, const EpiParams& pp,
                           int m, int n, int k, hipStream_t s) {
  if (p.kt_per_split % 2 == 0 && (k / BK) % 2 == 0)
    launch_mfma<EPI_PARTIAL, WGM, WGN, TI, TJ, true, STREAM_W>(a, w, nullptr, pp, m, n, k, s,
                                                               p.splits, p.kt_per_split);
  else
    launch_mfma<EPI_PARTIAL, WGM, WGN, TI, TJ, false, STREAM_W>(a, w, nullptr, pp, m, n, k, s,
                                                                p.splits, p.kt_per_split);
}

// the partial-sum GEMM of a split plan: fp32 planes part[splits][m][n]
static void launch_partials(const SplitPlan& p, const void* a, const void* w, float* part, int m,
                            int n, int k, hipStream_t s) {
  EpiParams pp{};
  pp.out = part;
  pp.ldo = n;
  // up to 64 rows are one row tile: each weight is read by one workgroup
  if (p.tile == 0) launch_partial<1, 4, 1, 1, true>(p, a, w, pp, m, n, k, s);
  else if (p.tile == 1) launch_partial<1, 4, 2, 1, true>(p, a, w, pp, m, n, k, s);
  else if (p.tile == 2) launch_partial<2, 2, 2, 2>(p, a, w, pp, m, n, k, s);
  else launch_partial<4, 2, 2, 4>(p, a, w, pp, m, n, k, s);
}

template <int EPI>
static void launch_split(const SplitPlan& p, const void* a, const void* w, const void* bias,
                         const EpiParams& ep, float* part, int m, int n, int k, hipStream_t s) {
  launch_partials(p, a, w, part, m, n, k, s);
  const int threads = m * (n / 4);
  hipLaunchKernelGGL(skinny_reduce_kernel<EPI>, dim3((threads + 255) / 256), dim3(256), 0, s,
                     part, p.splits, (const bf16*)bias, ep, m, n);
}

template <int EPI>
static void launch_typed(int dtype, const void* a, const void* w, const void* bias,
                         const EpiParams& ep, void* ws, size_t ws_bytes, int m, int n, int k,
                         hipStream_t s) {
  if (dtype == ORCA_BF16) {
    SplitPlan sp{};
    int v = plan_gemm(m, n, k, sp);
    if (v == 10) {
      if (ws && ws_bytes >= (size_t)sp.splits * m * n * sizeof(float)) {
        launch_split<EPI>(sp, a, w, bias, ep, static_cast<float*>(ws), m, n, k, s);
        return;
      }
      double c;
      v = best_tiled(m, n, c);   // no room for the partials: the best tiled launch
    }
    switch (v) {
      case 0: launch_mfma<EPI, 2, 2, 2, 2>(a, w, bias, ep, m, n, k, s); break;
      case 3: launch_mfma<EPI, 4, 2, 2, 4>(a, w, bias, ep, m, n, k, s); break;
      case 11:
        if ((k / BK) % 2 == 0 && (long)std::max(m, n) * k < (1L << 31)) {
          const int tiles_m = (m + 255) / 256, tiles_n = (n + 255) / 256;
          hipLaunchKernelGGL(gemm_ws_kernel<EPI>, dim3(tiles_m * tiles_n), dim3(WS_THREADS), 0, s,
                             (const bf16*)a, (const bf16*)w, (const bf16*)bias, ep, m, n, k,
                             tiles_m);
          break;
        }
        [[fallthrough]];   // odd K steps or offsets past 2^31: the 256 x 256 form
      case 14:
      case 15:
        if ((long)std::max(m, n) * k < (1L << 31)) {
          const int bn = v == 14 ? 256 : 192;
          const int tiles_m = (m + 255) / 256, tiles_n = (n + bn - 1) / bn;
          const bool k64 = env_int("ORCA_D4_K64", 0) != 0;
          auto kern = v == 14 ? (k64 ? gemm_d4_kernel<EPI, 4, 64> : gemm_d4_kernel<EPI, 4, 32>)
                              : (k64 ? gemm_d4_kernel<EPI, 3, 64> : gemm_d4_kernel<EPI, 3, 32>);
          hipLaunchKernelGGL(kern, dim3(tiles_m * tiles_n), dim3(W4_THREADS), 0, s,
                             (const bf16*)a, (const bf16*)w, (const bf16*)bias, ep, m, n, k,
                             tiles_m, raster_group(tiles_m));
          break;
        }
        v = v == 14 ? 12 : 13;   // offsets past 2^31: the register-staged forms' fallbacks
        [[fallthrough]];
      case 12:
      case 13:
        if ((v == 12 || v == 13) && w4_ok(m, n, k)) {
          const int bn = v == 12 ? 256 : 192;
          const int tiles_m = (m + 255) / 256, tiles = w4_tiles(m, n, bn);
          TileMap map{tiles_m, tiles, raster_group(tiles_m), 0, k / BK, 0};
          TailPlan t;
          const bool tail = tail_plan(tiles, k / BK, t) && ws &&
                            ws_bytes >= t.slots * 256 * bn * sizeof(float);
          if (tail) map.ntiles = tiles;
          auto kern = v == 12 ? gemm_w4_kernel<EPI, 4> : gemm_w4_kernel<EPI, 3>;
          const int n_dp = tail ? t.n_dp : tiles;
          // more than one round: one persistent workgroup per CU walks them
          if (n_dp > NUM_CU && env_int("ORCA_GEMM_PERSIST", 1)) map.persist = n_dp;
          hipLaunchKernelGGL(kern, dim3(map.persist ? NUM_CU : n_dp), dim3(W4_THREADS), 0, s,
                             (const bf16*)a, (const bf16*)w, (const bf16*)bias, ep, m, n, k, map);
          if (tail) {
            TileMap tm{tiles_m, tiles, map.group, t.n_dp, t.per, t.n_tail, 0, t.sk_kt};
            EpiParams pp{};
            pp.out = ws;
            auto pk = v == 12 ? gemm_w4_kernel<EPI_PARTIAL, 4> : gemm_w4_kernel<EPI_PARTIAL, 3>;
            hipLaunchKernelGGL(pk, t.sk_kt ? dim3(t.wgs) : dim3(t.n_tail, t.splits),
                               dim3(W4_THREADS), 0, s,
                               (const bf16*)a, (const bf16*)w, (const bf16*)bias, pp, m, n, k,
                               tm);
            auto rk = v == 12 ? tail_reduce_kernel<EPI, 256> : tail_reduce_kernel<EPI, 192>;
            hipLaunchKernelGGL(rk, dim3(t.n_tail, 16), dim3(256), 0, s,
                               static_cast<const float*>(ws), t.splits, tm, (const bf16*)bias,
                               ep, m, n);
          }
          break;
        }
        if (v == 13) {   // odd K steps or offsets past 2^31: the 256 x 192 form
          if ((k / BK) % 2 == 0) launch_mfma<EPI, 4, 2, 2, 3, true>(a, w, bias, ep, m, n, k, s);
          else launch_mfma<EPI, 4, 2, 2, 3>(a, w, bias, ep, m, n, k, s);
          break;
        }
        [[fallthrough]];
      case 6:
        if ((k / BK) % 2 == 0) launch_mfma<EPI, 4, 2, 2, 4, true>(a, w, bias, ep, m, n, k, s);
        else launch_mfma<EPI, 4, 2, 2, 4>(a, w, bias, ep, m, n, k, s);
        break;
      case 8:
        if ((k / BK) % 2 == 0) launch_mfma<EPI, 4, 2, 2, 3, true>(a, w, bias, ep, m, n, k, s);
        else launch_mfma<EPI, 4, 2, 2, 3>(a, w, bias, ep, m, n, k, s);
        break;
      default:  // 7, and the split-K choice when it does not apply
        if ((k / BK) % 2 == 0) launch_mfma<EPI, 2, 2, 2, 2, true>(a, w, bias, ep, m, n, k, s);
        else launch_mfma<EPI, 2, 2, 2, 2>(a, w, bias, ep, m, n, k, s);
        break;
    }
  } else {
    hipLaunchKernelGGL(gemm_f32_kernel<EPI>, dim3((n + 63) / 64, (m + 63) / 64), dim3(256), 0, s,
                       (const float*)a, (const float*)w, (const float*)bias, ep, m, n, k);
  }
}

hipError_t launch_linear(int dtype, int epilogue, const void* a, const void* w, const void* bias,
                         void* out, const QkvDest* qkv, int m, int n, int k, void* ws,
                         size_t ws_bytes, hipStream_t s) {
  if (m == 0) return hipSuccess;
  EpiParams ep{};
  ep.out = out;
  ep.ldo = n;
  if (qkv) ep.qkv = *qkv;
  switch (epilogue) {
    case ORCA_EPI_BIAS:
      launch_typed<ORCA_EPI_BIAS>(dtype, a, w, bias, ep, ws, ws_bytes, m, n, k, s);
      break;
    case ORCA_EPI_BIAS_GELU:
      launch_typed<ORCA_EPI_BIAS_GELU>(dtype, a, w, bias, ep, ws, ws_bytes, m, n, k, s);
      break;
    case ORCA_EPI_BIAS_RESID:
      launch_typed<ORCA_EPI_BIAS_RESID>(dtype, a, w, bias, ep, ws, ws_bytes, m, n, k, s);
      break;
    default: launch_typed<EPI_QKV>(dtype, a, w, bias, ep, ws, ws_bytes, m, n, k, s); break;
  }
  return hipGetLastError();
}

hipError_t launch_linear_resid_ln(int dtype, const void* a, const void* w, const void* bias,
                                  float* resid, int m, int n, int k, void* ws, size_t ws_bytes,
                                  const void* ln_g, const void* ln_b, void* ln_out, float eps,
                                  hipStream_t s, hipEvent_t after_gemm) {
  if (m == 0) return hipSuccess;
  SplitPlan sp{};
  if (dtype == ORCA_BF16 && plan_gemm(m, n, k, sp) == 10 && ws &&
      ws_bytes >= (size_t)sp.splits * m * n * sizeof(float)) {
    float* part = static_cast<float*>(ws);
    launch_partials(sp, a, w, part, m, n, k, s);
    const hipError_t e = after_gemm ? hipEventRecord(after_gemm, s) : hipGetLastError();
    if (e != hipSuccess) return e;
    const hipError_t f =
        launch_reduce_resid_ln(part, sp.splits, bias, resid, m, n, ln_g, ln_b, ln_out, eps, s);
    if (f != hipErrorNotSupported) return f;
    // row too wide for the fused kernel: the separate reduce, then the LN
    EpiParams ep{};
    ep.out = resid;
    ep.ldo = n;
    const int threads = m * (n / 4);
    hipLaunchKernelGGL(skinny_reduce_kernel<ORCA_EPI_BIAS_RESID>, dim3((threads + 255) / 256),
                       dim3(256), 0, s, part, sp.splits, (const bf16*)bias, ep, m, n);
  } else {
    const hipError_t e = launch_linear(dtype, ORCA_EPI_BIAS_RESID, a, w, bias, resid, nullptr, m,
                                       n, k, ws, ws_bytes, s);
    if (e != hipSuccess) return e;
    if (after_gemm) {
      const hipError_t f = hipEventRecord(after_gemm, s);
      if (f != hipSuccess) return f;
    }
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_layernorm(dtype, resid, ln_g, ln_b, ln_out, m, n, eps, s);
}

}  // namespace orca

// ------------------------------------------------- allocation-free Linear

// The split-K partial sums of orca_op_linear_noalloc.  Every GPU the library
// runs on holds its own copy until the process ends.  In host code the name
// stands for no device address: the address comes from hipGetSymbolAddress
// with the device current, once per device.
static __device__ __align__(256) unsigned char scratch[ORCA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex scratch_mu;
void* scratch_dev[MAX_DEVICES] = {};

// Address of the current device's copy of `scratch`.
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    scratch_dev[dev] = p;
  }
  *out = scratch_dev[dev];
  return hipSuccess;
}

}  // namespace

extern "C" orca_status orca_op_linear_noalloc(int32_t dtype, int32_t epilogue, const void* a,
                                              const void* w, const void* bias, void* out,
                                              int32_t m, int32_t n, int32_t k, void* stream) {
  orca::clear_error();
  ORCA_CHECK_ARG(dtype == ORCA_F32 || dtype == ORCA_BF16, "unknown dtype %d", dtype);
  ORCA_CHECK_ARG(epilogue >= ORCA_EPI_BIAS && epilogue <= ORCA_EPI_BIAS_RESID,
                 "unknown epilogue %d", epilogue);
  ORCA_CHECK_ARG(m >= 0 && n >= 64 && k >= 64, "shape m %d n %d k %d", m, n, k);
  if (n % 64 || k % 64) {
    orca::set_error("unsupported shape: n %d and k %d must be multiples of 64", n, k);
    return ORCA_ERR_UNSUPPORTED;
  }
  ORCA_CHECK_ARG(m == 0 || (a && w && bias && out), "NULL argument");
  if (m == 0) return ORCA_OK;
  const size_t need = orca::linear_workspace_bytes(dtype, m, n, k);
  const bool few_rows = orca::linear_plan_variant(dtype, m, n, k) == 10;
  if (need > ORCA_NOALLOC_SCRATCH_BYTES && few_rows) {
    orca::set_error("the split-K partial sums of m %d n %d k %d need %zu bytes; the static "
                    "scratch holds %zu (use orca_op_linear with a workspace)",
                    m, n, k, need, (size_t)ORCA_NOALLOC_SCRATCH_BYTES);
    return ORCA_ERR_UNSUPPORTED;
  }
  // a tiled problem whose split tail would not fit runs without it
  void* ws = nullptr;
  hipError_t e = need > ORCA_NOALLOC_SCRATCH_BYTES ? hipSuccess : scratch_address(&ws);
  if (e == hipSuccess)
    e = orca::launch_linear(dtype, epilogue, a, w, bias, out, nullptr, m, n, k, ws,
                            ws ? ORCA_NOALLOC_SCRATCH_BYTES : 0,
                            static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    orca::set_error("orca_op_linear_noalloc: %s", hipGetErrorString(e));
    return ORCA_ERR_HIP;
  }
  return ORCA_OK;
}
