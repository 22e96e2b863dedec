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
// lane group) accumulates the value rows.  Eight keys per lane group are in
// flight per loop trip, loaded with the non-temporal hint (each cached key
// and value is read once per layer).  The lane groups, then the four waves, are merged
// through shuffles and LDS into one (m, l, o[d]) partial per item; a second
// kernel merges the partials of a row and writes o at the row's own offset
// (the merge is index arithmetic: no copy).
//
// The pool keeps each slot's key row and value row next to each other
// ([heads][cap][2][d]), so a work item streams one contiguous range of
// 2 * keys * d elements rather than two ranges in two pools: with separate
// pools, the two streams of every workgroup measured 3-9% slower.
//
// HBM traffic of the split path per (row, head): 2 * keys * d * sizeof(T)
// bytes of K and V, read once.
#include <math.h>
#include <stdlib.h>

#include <algorithm>
#include <vector>

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
  constexpr int U = 8;
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

  // slot s of head h: key row at (h * cap + s) * 2D, its value row D later
  const size_t head_base = ((size_t)h * a.cap + (size_t)rq.kv_base) * 2 * D + e * VEC;
  const T* kb = (const T*)a.kv_pool + head_base;
  const T* vb = kb + D;

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
        // each cached key and value is read once per layer: stream them
        kr[u] = load_nt16(kb + (size_t)key * 2 * D);
        vr[u] = load_nt16(vb + (size_t)key * 2 * D);
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
    // one pass with a running max, four partials per trip, all their loads
    // issued before any is used (a clamped index re-reads the last partial
    // and is skipped): a loop trip per partial made each a round trip
    float mx = NEG_BIG, lt = 0.f, ot = 0.f;
    for (int i0 = 0; i0 < sr.item_count; i0 += 4) {
      float pm[4], pl[4], po[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const size_t pi =
            (size_t)(sr.item_begin + min(i0 + u, sr.item_count - 1)) * a.heads + h;
        pm[u] = a.part_ml[pi * 2];
        pl[u] = a.part_ml[pi * 2 + 1];
        po[u] = a.part_o[pi * D + t];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        // a select, not a branch: behind a branch the loads sink into it
        const bool on = i0 + u < sr.item_count;
        const float mn = fmaxf(mx, pm[u]);
        const float c0 = exp2f(mx - mn), c1 = exp2f(pm[u] - mn);
        lt = on ? lt * c0 + pl[u] * c1 : lt;
        ot = on ? ot * c0 + po[u] * c1 : ot;
        mx = on ? mn : mx;
      }
    }
    store_f32((T*)a.o + (size_t)sr.row * a.hidden + h * D + t, ot / lt);
  }
}

// ------------------------------------------------------------ prefill (MFMA)
//
// Initiation rows of a bf16 model: causal attention of a prompt over itself.
// A 256-thread workgroup takes one head and PREFILL_ROWS = 128 consecutive
// query positions of one request (32 per wave) and walks the request's keys
// 0 .. last query position in steps of BKV (64 or 32; see
// prefill_keys_per_step).  Each step's K and V rows are staged row-major in
// LDS (16-byte writes, two stages: the next step is written while this one
// is read).
//
// Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
// a lane then owns one query (its column) and 16 of the 32 keys of each
// MFMA tile, so the softmax max / sum need one cross-lane step (lane ^ 32).
// The probabilities feed O^T = V^T P^T straight from the score registers:
// a lane's eight keys of a 16-key PV step are the ones its score registers
// hold (keys 0-3 and 8-11 of the group for the lower half-wave, 4-7 and
// 12-15 for the upper), and V^T's operand is read in that key order with
// gfx950's transposing LDS read (ds_read_b64_tr_b16: each lane of a 16-lane
// group receives one column of a 4-key x 16-dim block whose rows the
// group's lanes address, four keys of one dim), so P never moves between
// lanes and V is never transposed in memory.
//
// Online softmax in base 2 with a running max and sum per query.  The
// running max is raised only when some query's block max exceeds it by more
// than PF_RESCALE_SLACK (then the accumulators are rescaled); otherwise the
// probabilities of the block are exp2 of at most that slack, well inside
// fp32 and bf16 range, and the final division by the row sum removes the
// offset exactly as it removes the usual one.  The row sums take the
// probabilities as rounded to bf16 for the PV product (a bf16 dot product
// with ones), so numerator and denominator see the same values.  The output
// tile is transposed through LDS so the [sum L, H] rows are written with
// 16-byte stores.
//
// K/V rows are fetched with buffer loads whose resource covers one step's
// keys and ends at the block's last key: rows past it read as zeros (their
// scores are masked), so no address is clamped per load.
constexpr float PF_RESCALE_SLACK = 8.0f;

typedef short s16x4_t __attribute__((ext_vector_type(4)));

// transposing LDS read: lane j of each 16-lane group gets element (j % 4)
// of the 4-element rows addressed by lanes 4k + (j % 16) / 4 of its group,
// k = 0..3
__device__ __forceinline__ s16x4_t lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4_t*)(p));
}

// a value of lane l and of lane l ^ 32 combined (gfx950's v_permlane32_swap
// hands each half-wave the other half's value)
__device__ __forceinline__ float halves_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D, int BKV, int WG_PER_CU>
__global__ __launch_bounds__(256, WG_PER_CU) void attn_prefill_kernel(AttnArgs a) {
  constexpr int BQ = PREFILL_ROWS;       // 128 queries: 32 per wave
  constexpr int NT = BKV / 32;           // 32-key score tiles per step
  constexpr int KLD = D + 8;             // K row stride (elements)
  // V row stride: rows 64 bytes apart modulo the 256-byte bank cycle, so a
  // transposing read's eight key rows (64 bytes each) fill the banks twice
  constexpr int VLD = D + 32;
  constexpr int OLD = D + 8;             // output staging row stride
  constexpr int K_ELEMS = BKV * KLD;
  constexpr int STAGE = BKV * (KLD + VLD);
  constexpr int O_ELEMS = BQ * OLD;
  constexpr int SMEM = 2 * STAGE > O_ELEMS ? 2 * STAGE : O_ELEMS;
  static_assert((VLD / 2) % 16 == 0 && ((VLD / 2) / 16) % 2 == 1, "V stride");
  __shared__ __attribute__((aligned(16))) uint16_t smem[SMEM];

  // workgroup i computes the tile and head of slot i (prefill_schedule)
  const PrefillSlot sl = a.pf_slots[blockIdx.x];
  const PrefillItem it = a.pf[sl.item];
  const int h = sl.head;
  const DevReq rq = a.reqs[it.req];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // the wave (uniform)
  const int half = lane >> 5, col = lane & 31;
  const size_t H = (size_t)a.hidden;

  // this lane's query: row qi of the prompt chunk, at absolute position
  // qpos = kv_len + qi (kv_len: prompt tokens cached by earlier chunks)
  const int qi = it.q0 + w * 32 + col;
  const int qpos = rq.kv_len + qi;
  const int qmin = rq.kv_len + it.q0 + w * 32;   // the wave's first query position
  const int qrow = rq.q_offset + min(qi, it.q1 - 1);
  bf16x8_t qf[D / 16];
  {
    const bf16* qp = (const bf16*)a.q + (size_t)qrow * H + h * D + half * 8;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qf[ks] = *reinterpret_cast<const bf16x8_t*>(qp + ks * 16);
  }
  f32x16_t o[D / 32];
#pragma unroll
  for (int dm = 0; dm < D / 32; ++dm)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dm][r] = 0.f;
  float m_run = NEG_BIG, l_run = 0.f;
  const float sc = LOG2E / sqrtf((float)D);

  // keys the block needs, and this wave (absolute positions, exclusive)
  const int kend = rq.kv_len + min(it.q1, it.q0 + BQ);
  // (a wave whose 32 rows all lie past the chunk's end computes nothing)
  const int kend_wave =
      it.q0 + w * 32 < it.q1 ? rq.kv_len + min(it.q1, it.q0 + w * 32 + 32) : 0;
  const bf16* kb =
      (const bf16*)a.kv_pool + ((size_t)h * a.cap + (size_t)rq.kv_base) * 2 * D;

  // K and V of the step after next are loaded into registers while the
  // current step runs on the MFMAs.  Thread tid loads 16 bytes of key rows
  // tid / (D/8) + (256 / (D/8)) i, at dims 8 (tid % (D/8)); the value row
  // follows the key row in the pool (instruction offset 2D bytes).
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int RPP = 256 / CPR;             // rows per pass of the workgroup
  constexpr int NL = BKV / RPP;              // passes per step (K and V each)
  static_assert(NL * RPP == BKV, "tile not divisible by threads");
  const int lrow = tid / CPR, lch = tid % CPR;
  typedef uint32_t Stage __attribute__((ext_vector_type(4 * NL)));
  typedef uint32_t U4 __attribute__((ext_vector_type(4)));
  Stage kreg, vreg;
  // the resource of a step covers its keys k0 .. min(k0 + BKV, kend) - 1
  // (none past kend; at most BKV rows, so its size never nears 2^31).  Its
  // size goes through readfirstlane: computed on the vector unit, it would
  // not be known to be uniform, and every load would then be wrapped in a
  // loop over the distinct resources of the wave (MI355X: 6% of the 13B
  // prompts' prefill time, 5% of the 175B-layer mix's).
#define ORCA_PF_LOAD(K0)                                                                     \
  {                                                                                          \
    const int k0_ = (K0);                                                                    \
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(                     \
        (void*)(kb + (size_t)k0_ * 2 * D), (short)0,                                         \
        __builtin_amdgcn_readfirstlane(max(0, min(kend - k0_, BKV)) * 2 * D * 2), 0x00020000); \
    _Pragma("unroll") for (int i = 0; i < NL; ++i) {                                         \
      const uint32_t off = (uint32_t)(((lrow + RPP * i) * 2 * D + lch * 8) * 2);             \
      const U4 tk = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);                    \
      const U4 tv = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 2 * D, 0, 0);            \
      kreg[4 * i] = tk.x; kreg[4 * i + 1] = tk.y; kreg[4 * i + 2] = tk.z; kreg[4 * i + 3] = tk.w; \
      vreg[4 * i] = tv.x; vreg[4 * i + 1] = tv.y; vreg[4 * i + 2] = tv.z; vreg[4 * i + 3] = tv.w; \
    }                                                                                        \
  }
#define ORCA_PF_STORE(BUF)                                                                   \
  {                                                                                          \
    uint16_t* const stK = smem + (BUF) * STAGE;                                              \
    uint16_t* const stV = stK + K_ELEMS;                                                     \
    _Pragma("unroll") for (int i = 0; i < NL; ++i) {                                         \
      *reinterpret_cast<uint4*>(&stK[(lrow + RPP * i) * KLD + lch * 8]) =                    \
          make_uint4(kreg[4 * i], kreg[4 * i + 1], kreg[4 * i + 2], kreg[4 * i + 3]);        \
      *reinterpret_cast<uint4*>(&stV[(lrow + RPP * i) * VLD + lch * 8]) =                    \
          make_uint4(vreg[4 * i], vreg[4 * i + 1], vreg[4 * i + 2], vreg[4 * i + 3]);        \
    }                                                                                        \
  }
  // this lane's transposing-read row: key 4 half + (lane % 16) / 4 of a
  // 16-key group, dims 16 ((lane / 16) % 2) + 4 (lane % 4) of a 32-dim block
  const int g16 = lane & 15;
  const int vtr = (4 * half + (g16 >> 2)) * VLD + 16 * ((lane >> 4) & 1) + 4 * (g16 & 3);
  const int kfr = col * KLD + half * 8;     // K fragment: key col, dims 8 half
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};

  ORCA_PF_LOAD(0)
  ORCA_PF_STORE(0)
  ORCA_PF_LOAD(BKV)
  __syncthreads();
  int cur = 0;
  for (int k0 = 0; k0 < kend; k0 += BKV, cur ^= 1) {
    // step k+1's K/V into the other stage: it was last read in step k-1,
    // which the barrier closing that step has ended for every wave
    if (k0 + BKV < kend) {
      ORCA_PF_STORE(cur ^ 1)
    }
    ORCA_PF_LOAD(k0 + 2 * BKV)
    if (k0 < kend_wave) {
      const uint16_t* sK = smem + cur * STAGE;
      const uint16_t* sV = sK + K_ELEMS;

      // S^T = K Q^T for keys k0 .. k0+63 (two 32-key tiles)
      f32x16_t s[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[t][r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const bf16x8_t kf =
              *reinterpret_cast<const bf16x8_t*>(&sK[kfr + 32 * t * KLD + ks * 16]);
          s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s[t], 0, 0, 0);
        }
      }
      // causal mask, only on blocks reaching past the wave's first query or
      // the last key (wave-uniform test); block max on the raw scores (the
      // scale is positive and folded into the exponent below), four
      // independent chains per lane
      float mq[4] = {NEG_BIG, NEG_BIG, NEG_BIG, NEG_BIG};
      if (k0 + BKV - 1 <= qmin && k0 + BKV <= kend) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) mq[r & 3] = fmaxf(mq[r & 3], s[t][r]);
      } else {
        // key k0 + 32 t + 8 (r / 4) + 4 half + r % 4 is visible when it is
        // at most min(qpos, kend - 1)
        const int lim = min(qpos, kend - 1) - k0 - 4 * half;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            s[t][r] = 32 * t + 8 * (r >> 2) + (r & 3) <= lim ? s[t][r] : NEG_BIG;
            mq[r & 3] = fmaxf(mq[r & 3], s[t][r]);
          }
      }
      const float mx = halves_max(fmaxf(fmaxf(mq[0], mq[1]), fmaxf(mq[2], mq[3]))) * sc;
      // every query sees key 0 in the first block, so m_run is finite from
      // then on; a masked score's exponent is far below it (p = 0)
      if (__any(mx > m_run + PF_RESCALE_SLACK)) {
        const float m_new = fmaxf(m_run, mx);
        const float corr = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= corr;
#pragma unroll
        for (int dm = 0; dm < D / 32; ++dm)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[dm][r] *= corr;
      }
      // exponents are <= PF_RESCALE_SLACK: the bare hardware exp2 (results
      // below 2^-126 flush to zero, which no sum can see)
      float lq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < 2 * NT; ++st) {
        const int t = st >> 1, rb = (st & 1) * 8;
        bf16x8_t pb;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          pb[j] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[t][rb + j], sc, -m_run));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bf16x2_t pp = {pb[2 * j], pb[2 * j + 1]};
          lq[j] = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, lq[j], false);
        }
        // O^T += V^T P^T over the 16 keys of this step (k0 + 16 st ..)
#pragma unroll
        for (int dm = 0; dm < D / 32; ++dm) {
          const uint16_t* vp = &sV[vtr + 16 * st * VLD + 32 * dm];
          const s16x4_t v0 = lds_read_tr16(vp);
          const s16x4_t v1 = lds_read_tr16(vp + 8 * VLD);
          const bf16x8_t vf =
              __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
          o[dm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb, o[dm], 0, 0, 0);
        }
      }
      l_run += (lq[0] + lq[1]) + (lq[2] + lq[3]);
    }
    __syncthreads();
  }

#undef ORCA_PF_LOAD
#undef ORCA_PF_STORE
  // normalise, transpose through LDS, write the rows
  const float l_tot = halves_sum(l_run);
  const float inv = 1.f / l_tot;
  __syncthreads();
  uint16_t* sO = smem;
#pragma unroll
  for (int dm = 0; dm < D / 32; ++dm)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int d = dm * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
      sO[(w * 32 + col) * OLD + d] = f32_to_bf16_bits(o[dm][r] * inv);
    }
  __syncthreads();
  for (int c = tid; c < BQ * (D / 8); c += 256) {
    const int ql = c / (D / 8), ch = c % (D / 8);
    const int qp = it.q0 + ql;
    if (qp < it.q1)
      *reinterpret_cast<uint4*>((bf16*)a.o + (size_t)(rq.q_offset + qp) * H + h * D + ch * 8) =
          *reinterpret_cast<const uint4*>(&sO[ql * OLD + ch * 8]);
  }
}

// Prefill form: 64-key steps with two workgroups per CU (~200 registers a
// lane), or 32-key steps with three (~165 registers; 38 KB of LDS each).
// Three per CU hide more of a step's latency but double the steps of every
// tile, so they pay when the tiles are many (throughput-bound) and not when
// the longest tile's chain of steps bounds the launch.  Measured (kernel
// trace, MI355X): the 175B-layer prompt mix (8 prompts, 96 heads, 2,976
// tiles) 110.6 -> 102 us with 32-key steps; two 1,024-token 13B prompts (40
// heads, 640 tiles) 38.7 -> 40.5 us.  Above two rounds of two-per-CU slots
// the 32-key form is taken.  ORCA_PF_KEYS (32 or 64) pins one, for tests.
int prefill_keys_per_step(int heads, int n_pf) {
  if (const char* v = getenv("ORCA_PF_KEYS")) return atoi(v) == 32 ? 32 : 64;
  return (long)heads * n_pf > 2L * 2 * 256 ? 32 : 64;
}

// Order of a prefill launch's workgroups.  MI355X hands workgroup i to XCD
// i % 8, each XCD with its own 4 MB L2, and every tile of one (request,
// head) reads that head's keys and values from position 0 up.
//  * Longest-first (up to two rounds of two-per-CU workgroups): workgroup i
//    takes tile i / heads of the longest-first tile list and head i % heads,
//    so the launch ends with its longest chain of key steps.
//  * Grouped (more rounds): the (request, head) groups go, the requests with
//    the most work first, to the XCD holding the fewest workgroups so far,
//    each group's tiles one after another, so they run together and share
//    their key/value reads through that XCD's L2; the lists are then evened
//    out (XCD x takes the workgroups x, x + 8, ...).  MI355X, kernel trace:
//    the 175B-layer prompt mix (8 prompts, 96 heads, 2,976 workgroups)
//    103 -> 95 us, L2 fills 241 -> 122 MiB; over fewer rounds the groups
//    that start last end the launch late (two 1,024-token 13B prompts, 640
//    workgroups: 38.7 us longest-first, 48.9 grouped).
bool prefill_grouped(int heads, int n_pf) {
  if (const char* v = getenv("ORCA_PF_ORDER")) return atoi(v) == 1;
  return (long)heads * n_pf > 2L * 2 * 256;
}

void prefill_schedule(const DevReq* reqs, int n_reqs, PrefillItem* pf, int n_pf, int heads,
                      PrefillSlot* slots) {
  // causal tiles cost ~ their last key position (cached prefix + last query)
  auto end = [&](const PrefillItem& t) { return int64_t(reqs[t.req].kv_len) + t.q1; };
  std::sort(pf, pf + n_pf, [&](const PrefillItem& a, const PrefillItem& b) {
    const int64_t ea = end(a), eb = end(b);
    return ea != eb ? ea > eb : (a.req != b.req ? a.req < b.req : a.q0 < b.q0);
  });
  const int n = n_pf * heads;
  if (!prefill_grouped(heads, n_pf)) {
    for (int i = 0; i < n; ++i) slots[i] = PrefillSlot{i / heads, i % heads};
    return;
  }
  constexpr int NX = 8;   // XCDs
  std::vector<std::vector<int>> tiles(n_reqs);
  std::vector<int64_t> work(n_reqs, 0);
  for (int k = 0; k < n_pf; ++k) {
    tiles[pf[k].req].push_back(k);   // longest first
    work[pf[k].req] += end(pf[k]);
  }
  std::vector<int> order;
  for (int r = 0; r < n_reqs; ++r)
    if (!tiles[r].empty()) order.push_back(r);
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return work[a] > work[b]; });
  std::vector<PrefillSlot> xs[NX];
  int64_t xw[NX] = {};
  for (int r : order)
    for (int h = 0; h < heads; ++h) {
      int x = 0;
      for (int y = 1; y < NX; ++y)
        if (xs[y].size() < xs[x].size() || (xs[y].size() == xs[x].size() && xw[y] < xw[x])) x = y;
      for (int k : tiles[r]) xs[x].push_back(PrefillSlot{k, h});
      xw[x] += work[r];
    }
  // even out the lists: XCD x takes the n / 8 (+1 for x < n % 8)
  // workgroups x, x + 8, ...; surplus tiles (the shortest of the last
  // groups) move to the XCDs short of theirs
  std::vector<PrefillSlot> spill;
  for (int x = 0; x < NX; ++x)
    while ((int)xs[x].size() > n / NX + (x < n % NX)) {
      spill.push_back(xs[x].back());
      xs[x].pop_back();
    }
  for (int x = 0; x < NX; ++x) {
    const int cnt = n / NX + (x < n % NX);
    while ((int)xs[x].size() < cnt) {
      xs[x].push_back(spill.back());
      spill.pop_back();
    }
    for (int j = 0; j < cnt; ++j) slots[x + NX * j] = xs[x][j];
  }
}

// Residency of the split-KV kernel.  Its registers allow four to five
// 256-thread workgroups per CU, but the cache streams faster with two: fewer
// K/V streams at once per HBM channel (measured: two per CU +0.7% at the
// 175B layer shape, +2.6% at 13B, +3.5% on a 64-request decode batch; one per
// CU 12-20% slower).  The launch reserves enough LDS (unused) that only two
// fit in a CU's 160 KB.
constexpr unsigned SPLIT_LDS_RESERVE = 60 * 1024;

template <typename T, int D>
static void launch_split(const AttnArgs& a, hipStream_t s) {
  if constexpr (sizeof(T) == 2) {
    if (a.n_pf > 0) {
      if (prefill_keys_per_step(a.heads, a.n_pf) == 32)
        hipLaunchKernelGGL((attn_prefill_kernel<D, 32, 3>), dim3(a.heads * a.n_pf), dim3(256), 0, s,
                           a);
      else
        hipLaunchKernelGGL((attn_prefill_kernel<D, 64, 2>), dim3(a.heads * a.n_pf), dim3(256), 0, s,
                           a);
    }
  }
  if (a.n_items == 0) return;
  hipLaunchKernelGGL((attn_split_kernel<T, D>), dim3(a.n_items, a.heads), dim3(256),
                     SPLIT_LDS_RESERVE, s, a);
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
