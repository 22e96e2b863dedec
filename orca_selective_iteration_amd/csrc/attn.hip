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
// 0 .. last query position in steps of 64, staging each K step (row-major)
// and V step (transposed to [d][key]) in LDS.  Scores are computed
// transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: a lane then owns
// one query (its column) and 16 of the 32 keys of each MFMA tile, so the
// softmax max / sum need one cross-lane step (lane ^ 32).  The probabilities
// feed O^T = V^T P^T straight from the score registers: the keys of the
// PV MFMA's k-dimension are taken in the order in which the score tile
// left them in the lanes, and V^T stores the keys of every 16-key group in
// that order (keys 4-7 and 8-11 swapped), so a lane's eight keys are one
// 16-byte LDS read and P never moves between lanes.  Online softmax in base 2 with a running max
// and sum per query; the output tile is transposed through LDS so the
// [sum L, H] rows are written with 16-byte stores.
template <int D>
__global__ __launch_bounds__(256, 2) void attn_prefill_kernel(AttnArgs a) {
  constexpr int BQ = PREFILL_ROWS;       // 128 queries: 32 per wave
  constexpr int BKV = 64;                // keys per step
  constexpr int KLD = D + 8;             // K row stride (elements)
  constexpr int VLD = BKV + 8;           // V^T row stride
  constexpr int OLD = D + 8;             // output staging row stride
  constexpr int KV_ELEMS = BKV * KLD + D * VLD;
  constexpr int O_ELEMS = BQ * OLD;
  // two K/V stages (the next step is written while this one is read)
  constexpr int SMEM = 2 * KV_ELEMS > O_ELEMS ? 2 * KV_ELEMS : O_ELEMS;
  __shared__ __attribute__((aligned(16))) uint16_t smem[SMEM];

  // grid (heads, items): all heads of the first (longest) item go first
  const PrefillItem it = a.pf[blockIdx.y];
  const int h = blockIdx.x;
  const DevReq rq = a.reqs[it.req];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
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
  const int kend_wave = rq.kv_len + min(it.q1, it.q0 + w * 32 + 32);
  const size_t head_base = ((size_t)h * a.cap + (size_t)rq.kv_base) * 2 * D;
  const bf16* kb = (const bf16*)a.kv_pool + head_base;
  const bf16* vb = kb + D;   // each slot's value row follows its key row

  // K and V of the next 64-key step are loaded into registers while the
  // current step runs on the MFMAs (16-byte loads; keys past the block's
  // last one re-read it, so the loads never sit behind a branch)
  constexpr int NL = BKV * (D / 8) / 256;   // 16-byte loads per thread, K and V each
  static_assert(NL * 256 == BKV * (D / 8) && NL * 4 == D / 8, "tile not divisible by threads");
  // vector-typed staging (not arrays) keeps the prefetch in registers
  typedef uint32_t Stage __attribute__((ext_vector_type(4 * NL)));
  Stage kreg, vreg;
  const int vkey = tid & 63;
  // V^T column of key pair (vkey & ~1): bits 2 and 3 of the key swapped
  // inside its 16-key group, the order in which a lane's P^T fragment holds
  // its keys (4 half + 0..3, then 8 + 4 half + 0..3), so the lane's eight
  // keys are one 16-byte read
  const int vcol = (vkey & ~15) | (vkey & 2) | ((vkey & 4) << 1) | ((vkey & 8) >> 1);
  // byte selectors of v_perm_b32 (bytes 0-3: second operand, 4-7: first):
  // even key lanes take (own.lo16, neighbour.lo16), odd ones
  // (neighbour.hi16, own.hi16)
  const uint32_t vsel = (vkey & 1) ? 0x03020706u : 0x05040100u;
#define ORCA_PF_LOAD(K0)                                                                     \
  _Pragma("unroll") for (int i = 0; i < NL; ++i) {                                           \
    const int c = tid + 256 * i, key = c / (D / 8), ch = c % (D / 8);                        \
    const uint4 tk = *reinterpret_cast<const uint4*>(                                        \
        kb + (size_t)min((K0) + key, kend - 1) * 2 * D + ch * 8);                            \
    const uint4 tv = *reinterpret_cast<const uint4*>(                                        \
        vb + (size_t)min((K0) + vkey, kend - 1) * 2 * D + ((tid >> 6) + 4 * i) * 8);         \
    kreg[4 * i] = tk.x; kreg[4 * i + 1] = tk.y; kreg[4 * i + 2] = tk.z; kreg[4 * i + 3] = tk.w; \
    vreg[4 * i] = tv.x; vreg[4 * i + 1] = tv.y; vreg[4 * i + 2] = tv.z; vreg[4 * i + 3] = tv.w; \
  }
  // V^T: this lane holds dims d, d+1 of key vkey in each word; with the
  // neighbouring key's word (lane ^ 1, a DPP move) an even lane writes row d
  // (its own low half, then the neighbour's) and an odd lane row d+1 (the
  // neighbour's high half, then its own), two consecutive keys per 32-bit
  // store: one byte permute with a per-lane selector (a select between the
  // two forms compiled to a divergent branch)
#define ORCA_PF_STORE(BUF)                                                                   \
  {                                                                                          \
    uint16_t* const stK = smem + (BUF) * KV_ELEMS;                                           \
    uint16_t* const stV = stK + BKV * KLD;                                                   \
    _Pragma("unroll") for (int i = 0; i < NL; ++i) {                                         \
      const int c = tid + 256 * i, key = c / (D / 8), ch = c % (D / 8);                      \
      *reinterpret_cast<uint4*>(&stK[key * KLD + ch * 8]) =                                  \
          make_uint4(kreg[4 * i], kreg[4 * i + 1], kreg[4 * i + 2], kreg[4 * i + 3]);        \
      const int vch = (tid >> 6) + 4 * i;                                                    \
      _Pragma("unroll") for (int j = 0; j < 4; ++j) {                                        \
        const uint32_t wv = vreg[4 * i + j];                                                 \
        const uint32_t nb =                                                                  \
            (uint32_t)__builtin_amdgcn_update_dpp(0, (int)wv, 0xB1, 0xF, 0xF, false);       \
        *reinterpret_cast<uint32_t*>(&stV[(vch * 8 + 2 * j + (vkey & 1)) * VLD + vcol]) =    \
            __builtin_amdgcn_perm(nb, wv, vsel);                                             \
      }                                                                                      \
    }                                                                                        \
  }
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
    const uint16_t* sK = smem + cur * KV_ELEMS;
    const uint16_t* sV = sK + BKV * KLD;

    // S^T = K Q^T for keys k0 .. k0+63 (two 32-key tiles)
    f32x16_t s[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[t][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8_t kf =
            *reinterpret_cast<const bf16x8_t*>(&sK[(32 * t + col) * KLD + ks * 16 + half * 8]);
        s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s[t], 0, 0, 0);
      }
    }
    // causal mask, only on blocks reaching past the wave's first query or
    // the last key (wave-uniform test); running max on the raw scores, the
    // scale folded into the exponent below
    // (the max and the sum below run as four independent chains, not one
    // 32-deep dependent chain per lane)
    float mq[4] = {NEG_BIG, NEG_BIG, NEG_BIG, NEG_BIG};
    if (k0 + BKV - 1 <= qmin && k0 + BKV <= kend) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) mq[r & 3] = fmaxf(mq[r & 3], s[t][r]);
    } else {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * t + 8 * (r >> 2) + 4 * half + (r & 3);
          const bool vis = key <= qpos && key < kend;
          s[t][r] = vis ? s[t][r] : NEG_BIG;
          mq[r & 3] = fmaxf(mq[r & 3], s[t][r]);
        }
    }
    float mx = fmaxf(fmaxf(mq[0], mq[1]), fmaxf(mq[2], mq[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // every query sees key 0 in the first block, so m_run is finite from
    // then on and a masked score's exponent is far below it (p = 0)
    // exponents are <= 0 here: the bare hardware exp2 (exact at 0; results
    // below 2^-126 of the running max flush to zero, which no sum can see)
    // instead of exp2f's range fix-up, five more instructions per score
    const float m_new = fmaxf(m_run, mx * sc);
    const float corr = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    l_run *= corr;
    // once the running maxima settle, most steps leave every query's max
    // unchanged (corr == 1): skip the rescale of the output accumulators
    if (__any(corr != 1.f)) {
#pragma unroll
      for (int dm = 0; dm < D / 32; ++dm)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dm][r] *= corr;
    }
    float lq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[t][r], sc, -m_new));
        s[t][r] = p;
        lq[r & 3] += p;
      }
    l_run += (lq[0] + lq[1]) + (lq[2] + lq[3]);
    // O^T += V^T P^T, 16 keys per MFMA step
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int t = st >> 1, rb = (st & 1) * 8;
      bf16x8_t pb;
      {
        uint32_t pk[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) pk[j] = pack_bf16x2(s[t][rb + 2 * j], s[t][rb + 2 * j + 1]);
        pb = *reinterpret_cast<const bf16x8_t*>(pk);
      }
#pragma unroll
      for (int dm = 0; dm < D / 32; ++dm) {
        const bf16x8_t vf = *reinterpret_cast<const bf16x8_t*>(
            &sV[(dm * 32 + col) * VLD + 16 * st + 8 * half]);
        o[dm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb, o[dm], 0, 0, 0);
      }
    }
    }
    __syncthreads();
  }

#undef ORCA_PF_LOAD
#undef ORCA_PF_STORE
  // normalise, transpose through LDS, write the rows
  const float l_tot = l_run + __shfl_xor(l_run, 32);
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
    if (a.n_pf > 0)
      hipLaunchKernelGGL((attn_prefill_kernel<D>), dim3(a.heads, a.n_pf), dim3(256), 0, s, a);
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
