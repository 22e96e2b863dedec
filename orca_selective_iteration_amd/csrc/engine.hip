// The engine behind orca_iteration: descriptor validation, the per-iteration
// metadata (one asynchronous copy from a pinned ring), and the layer loop
// that launches the gfx950 kernels on the caller's stream.
//
// garden.houmin.site/infra/orca 3.1.1: the scheduler hands the engine one
// iteration of a selected batch; 3.1.2: non-attention operations run on the
// flattened [sum L, H] matrix, attention per request (split / merge are
// index arithmetic here).  unpurerationalist.github.io ORCA notes 4.1: the
// engine receives per request its token index and phase, and the host never
// waits for the GPU to hand over this metadata.  0h-n0.github.io digest,
// implementation notes: the K/V pool is allocated once, an index table
// records each request's slots (here: kv_base + position).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstdint>
#include <cstring>
#include <new>
#include <utility>
#include <vector>

#include "kernels.h"
#include "kv.h"
#include "orca.h"
#include "status.h"

using namespace orca;

namespace {

constexpr size_t ALIGN = 256;
constexpr int NSLOT = 4;

size_t align_up(size_t v) { return (v + ALIGN - 1) / ALIGN * ALIGN; }
size_t dsize(int dtype) { return dtype == ORCA_BF16 ? 2 : 4; }

bool head_dim_ok(int dtype, int d) {
  if (dtype == ORCA_BF16) return d == 64 || d == 128;
  return d == 16 || d == 32 || d == 64 || d == 128;
}

}  // namespace

struct orca_ctx {
  orca_model_desc desc{};
  std::vector<orca_layer_weights> layers;
  void* kv_pool = nullptr;   // [layers][heads][cap][2][d]
  const orca_kv* kv = nullptr;
  int32_t max_rows = 0, max_reqs = 0;
  int64_t max_items = 0, max_pf = 0;
  int device = 0;
  // workspace layout
  size_t off_resid = 0, off_a = 0, off_q = 0, off_o = 0, off_f = 0;
  size_t off_part_o = 0, off_part_ml = 0, off_meta = 0, ws_bytes = 0, meta_bytes = 0;
  size_t off_gpart = 0, gpart_bytes = 0;   // split-K partial sums of the few-rows Linear path
  // pinned staging ring for the metadata
  void* staging[NSLOT] = {};
  hipEvent_t ev[NSLOT] = {};
  bool ev_live[NSLOT] = {};
  int slot = 0;
  std::vector<std::pair<int64_t, int64_t>> ranges;   // scratch for validation
  // timing of one step of every layer (orca_time_step): events [layer][2]
  int probe_step = -1;
  bool probe_recorded = false;
  std::vector<hipEvent_t> probe_ev;

  // one layer of the pool: [heads][cap][2][d]
  size_t layer_pool_elems() const {
    return (size_t)desc.heads * (size_t)desc.kv_capacity * 2 * (size_t)(desc.hidden / desc.heads);
  }
};

namespace {

// Host-side plan of one iteration, written straight into a pinned slot.
struct Plan {
  DevReq* reqs;
  int32_t* row_dst;
  SplitItem* items;
  SplitRow* srows;
  PrefillItem* pf;
  PrefillSlot* slots;
  int n_reqs = 0, rows = 0, n_items = 0, n_srows = 0, n_pf = 0;
  size_t off_reqs = 0, off_row_dst = 0, off_items = 0, off_srows = 0, off_pf = 0, off_slots = 0,
         bytes = 0;
};

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// bf16 initiation rows take the MFMA prefill kernel; every other row the
// split-KV kernel.
bool uses_prefill(const orca_ctx* c, const orca_req_desc& r) {
  return c->desc.dtype == ORCA_BF16 && r.phase == ORCA_INITIATION;
}

// Validates the descriptors; on success returns ORCA_OK and the row count.
orca_status validate(orca_ctx* c, const orca_req_desc* reqs, int32_t n, int32_t* rows_out,
                     int64_t* items_out, int64_t* pf_out) {
  ORCA_CHECK_ARG(n >= 0 && n <= c->max_reqs, "batch of %d requests (max_reqs %d)", n,
                 c->max_reqs);
  ORCA_CHECK_ARG(n == 0 || reqs != nullptr, "reqs is NULL");
  int64_t off = 0, items = 0, pf = 0;
  c->ranges.clear();
  for (int i = 0; i < n; ++i) {
    const orca_req_desc& r = reqs[i];
    ORCA_CHECK_ARG(r.q_offset == off, "request %d: q_offset %d, expected %lld (contiguous)", i,
                   r.q_offset, (long long)off);
    ORCA_CHECK_ARG(r.q_len >= 1, "request %d: q_len %d < 1", i, r.q_len);
    ORCA_CHECK_ARG(r.kv_len >= 0, "request %d: kv_len %d < 0", i, r.kv_len);
    if (r.phase != ORCA_INITIATION) {
      ORCA_CHECK_ARG(r.phase == ORCA_INCREMENT, "request %d: unknown phase %d", i, r.phase);
      ORCA_CHECK_ARG(r.kv_len >= 1, "request %d: increment without a cache", i);
      ORCA_CHECK_ARG(r.q_len == 1, "request %d: increment with q_len %d", i, r.q_len);
    }
    const int64_t lo = r.kv_base, hi = r.kv_base + int64_t(r.kv_len) + r.q_len;
    ORCA_CHECK_ARG(lo >= 0 && hi <= c->desc.kv_capacity,
                   "request %d: slots [%lld, %lld) outside the pool of %lld", i, (long long)lo,
                   (long long)hi, (long long)c->desc.kv_capacity);
    if (c->kv)
      ORCA_CHECK_ARG(c->kv->covers(lo, hi), "request %d: slots [%lld, %lld) are not inside one "
                     "K/V reservation", i, (long long)lo, (long long)hi);
    c->ranges.emplace_back(lo, hi);
    off += r.q_len;
    if (uses_prefill(c, r)) {
      pf += ceil_div(r.q_len, PREFILL_ROWS);
    } else {
      for (int j = 0; j < r.q_len; ++j) items += ceil_div(int64_t(r.kv_len) + j + 1, SPLIT_CHUNK);
    }
  }
  ORCA_CHECK_ARG(off <= c->max_rows, "batch of %lld rows (max_rows %d)", (long long)off,
                 c->max_rows);
  std::sort(c->ranges.begin(), c->ranges.end());
  for (size_t i = 1; i < c->ranges.size(); ++i)
    ORCA_CHECK_ARG(c->ranges[i - 1].second <= c->ranges[i].first,
                   "two requests use overlapping K/V slots near %lld",
                   (long long)c->ranges[i].first);
  ORCA_CHECK_ARG(items <= c->max_items && pf <= c->max_pf, "batch needs %lld + %lld attention "
                 "work items, the workspace holds %lld + %lld", (long long)items, (long long)pf,
                 (long long)c->max_items, (long long)c->max_pf);
  *rows_out = int32_t(off);
  *items_out = items;
  *pf_out = pf;
  return ORCA_OK;
}

// Lays the plan out in `buf` (packed, 16-byte aligned sections).
void build_plan(const orca_ctx* c, const orca_req_desc* reqs, int32_t n, int32_t rows,
                int64_t n_items, int64_t n_pf, char* buf, Plan& p) {
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = (o + bytes + 15) / 16 * 16;
    return at;
  };
  p.off_reqs = take(sizeof(DevReq) * n);
  p.off_row_dst = take(sizeof(int32_t) * rows);
  p.off_items = take(sizeof(SplitItem) * n_items);
  p.off_srows = take(sizeof(SplitRow) * rows);
  p.off_pf = take(sizeof(PrefillItem) * n_pf);
  p.off_slots = take(sizeof(PrefillSlot) * n_pf * c->desc.heads);
  p.bytes = o;
  p.reqs = reinterpret_cast<DevReq*>(buf + p.off_reqs);
  p.row_dst = reinterpret_cast<int32_t*>(buf + p.off_row_dst);
  p.items = reinterpret_cast<SplitItem*>(buf + p.off_items);
  p.srows = reinterpret_cast<SplitRow*>(buf + p.off_srows);
  p.pf = reinterpret_cast<PrefillItem*>(buf + p.off_pf);
  p.slots = reinterpret_cast<PrefillSlot*>(buf + p.off_slots);
  p.n_reqs = n;
  p.rows = rows;
  int ni = 0, ns = 0, np = 0;
  for (int i = 0; i < n; ++i) {
    const orca_req_desc& r = reqs[i];
    p.reqs[i] = DevReq{r.q_offset, r.q_len, r.kv_len, r.phase, r.kv_base};
    const bool pre = uses_prefill(c, r);
    if (pre)
      for (int q0 = 0; q0 < r.q_len; q0 += PREFILL_ROWS)
        p.pf[np++] = PrefillItem{i, q0, std::min(r.q_len, q0 + PREFILL_ROWS), 0};
    for (int j = 0; j < r.q_len; ++j) {
      const int row = r.q_offset + j;
      const int64_t pos = int64_t(r.kv_len) + j;
      p.row_dst[row] = int32_t(r.kv_base + pos);
      if (pre) continue;
      const int keys = int(pos + 1);
      const int chunks = int(ceil_div(keys, SPLIT_CHUNK));
      p.srows[ns++] = SplitRow{row, ni, chunks, i};
      for (int ch = 0; ch < chunks; ++ch)
        p.items[ni++] = SplitItem{row, i, ch * SPLIT_CHUNK, std::min(keys, (ch + 1) * SPLIT_CHUNK)};
    }
  }
  p.n_items = ni;
  p.n_srows = ns;
  p.n_pf = np;
  // the tiles longest-first and the workgroup order of the prefill launch
  prefill_schedule(p.reqs, n, p.pf, np, c->desc.heads, p.slots);
}

orca_status hip_fail(hipError_t e, const char* what) {
  set_error("%s: %s", what, hipGetErrorString(e));
  return ORCA_ERR_HIP;
}

#define HIP_TRY(expr, what)                        \
  do {                                             \
    hipError_t _e = (expr);                        \
    if (_e != hipSuccess) return hip_fail(_e, what); \
  } while (0)

// Validates, stages and uploads the metadata; fills device-side pointers.
orca_status stage(orca_ctx* c, const orca_req_desc* reqs, int32_t n, char* ws, hipStream_t s,
                  Plan& p, AttnArgs& aa) {
  int32_t rows = 0;
  int64_t n_items = 0, n_pf = 0;
  orca_status st = validate(c, reqs, n, &rows, &n_items, &n_pf);
  if (st != ORCA_OK) return st;
  const int slot = c->slot;
  c->slot = (c->slot + 1) % NSLOT;
  if (c->ev_live[slot]) HIP_TRY(hipEventSynchronize(c->ev[slot]), "metadata ring wait");
  char* host = static_cast<char*>(c->staging[slot]);
  build_plan(c, reqs, n, rows, n_items, n_pf, host, p);
  char* dev = ws + c->off_meta;
  if (p.bytes > 0) {
    HIP_TRY(hipMemcpyAsync(dev, host, p.bytes, hipMemcpyHostToDevice, s), "metadata upload");
    HIP_TRY(hipEventRecord(c->ev[slot], s), "metadata event");
    c->ev_live[slot] = true;
  }
  const orca_model_desc& d = c->desc;
  aa = AttnArgs{};
  aa.dtype = d.dtype;
  aa.hidden = d.hidden;
  aa.heads = d.heads;
  aa.head_dim = d.hidden / d.heads;
  aa.cap = d.kv_capacity;
  aa.reqs = reinterpret_cast<const DevReq*>(dev + p.off_reqs);
  aa.items = reinterpret_cast<const SplitItem*>(dev + p.off_items);
  aa.n_items = p.n_items;
  aa.srows = reinterpret_cast<const SplitRow*>(dev + p.off_srows);
  aa.n_srows = p.n_srows;
  aa.pf = reinterpret_cast<const PrefillItem*>(dev + p.off_pf);
  aa.pf_slots = reinterpret_cast<const PrefillSlot*>(dev + p.off_slots);
  aa.n_pf = p.n_pf;
  aa.part_o = reinterpret_cast<float*>(ws + c->off_part_o);
  aa.part_ml = reinterpret_cast<float*>(ws + c->off_part_ml);
  return ORCA_OK;
}

}  // namespace

extern "C" {

orca_status orca_create(const orca_model_desc* desc, const orca_layer_weights* layers,
                        void* kv_pool, const orca_kv* kv, int32_t max_rows,
                        int32_t max_reqs, orca_ctx** out) {
  ORCA_CHECK_ARG(desc && layers && kv_pool && out, "orca_create: NULL argument");
  const orca_model_desc& d = *desc;
  ORCA_CHECK_ARG(d.dtype == ORCA_F32 || d.dtype == ORCA_BF16, "unknown dtype %d", d.dtype);
  ORCA_CHECK_ARG(d.layers >= 1 && d.hidden >= 64 && d.heads >= 1 && d.ffn >= 64,
                 "bad shape layers %d hidden %d heads %d ffn %d", d.layers, d.hidden, d.heads,
                 d.ffn);
  ORCA_CHECK_ARG(d.hidden % d.heads == 0, "hidden %d not divisible by heads %d", d.hidden,
                 d.heads);
  ORCA_CHECK_ARG(d.ln_eps > 0.f, "ln_eps must be > 0");
  ORCA_CHECK_ARG(d.kv_capacity >= 1 && d.kv_capacity < (int64_t(1) << 31),
                 "kv_capacity %lld out of range", (long long)d.kv_capacity);
  ORCA_CHECK_ARG(max_rows >= 1 && max_reqs >= 1, "max_rows / max_reqs must be >= 1");
  ORCA_CHECK_ARG(!kv || kv->capacity == d.kv_capacity, "allocator capacity %lld != pool %lld",
                 (long long)(kv ? kv->capacity : 0), (long long)d.kv_capacity);
  if (d.hidden % 64 || d.ffn % 64 || d.hidden > 12288 || !head_dim_ok(d.dtype, d.hidden / d.heads)) {
    set_error("unsupported shape: hidden %d ffn %d head_dim %d", d.hidden, d.ffn,
              d.hidden / d.heads);
    return ORCA_ERR_UNSUPPORTED;
  }
  for (int l = 0; l < d.layers; ++l) {
    const orca_layer_weights& w = layers[l];
    ORCA_CHECK_ARG(w.ln1_g && w.ln1_b && w.w_qkv && w.b_qkv && w.w_o && w.b_o && w.ln2_g &&
                   w.ln2_b && w.w_1 && w.b_1 && w.w_2 && w.b_2, "layer %d: NULL weight", l);
  }
  auto* c = new (std::nothrow) orca_ctx;
  ORCA_CHECK_ARG(c != nullptr, "out of host memory");
  c->desc = d;
  c->layers.assign(layers, layers + d.layers);
  c->kv_pool = kv_pool;
  c->kv = kv;
  c->max_rows = max_rows;
  c->max_reqs = max_reqs;
  // split-KV items: a row with `keys` keys yields ceil(keys / SPLIT_CHUNK).
  // bf16: only increment rows take this path, one per request over disjoint
  // pool ranges, so the keys of all of them add up to at most the capacity.
  // fp32: every row does, and the rows of one prompt chunk share a range;
  // each row has at most min(capacity, max_rows + its cached prefix) keys.
  c->max_items = int64_t(max_rows) + d.kv_capacity / SPLIT_CHUNK + 1;
  if (d.dtype == ORCA_F32)
    c->max_items = int64_t(max_rows) * (1 + d.kv_capacity / SPLIT_CHUNK) + 1;
  c->max_pf = d.dtype == ORCA_BF16 ? int64_t(max_rows) / PREFILL_ROWS + max_reqs : 0;
  const size_t R = max_rows, H = d.hidden, F = d.ffn, s = dsize(d.dtype);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  c->off_resid = take(R * H * 4);
  c->off_a = take(R * H * s);
  c->off_q = take(R * H * s);
  c->off_o = take(R * H * s);
  c->off_f = take(R * F * s);
  c->off_part_o = take(size_t(c->max_items) * H * 4);
  c->off_part_ml = take(size_t(c->max_items) * d.heads * 2 * 4);
  // split-K partial sums of the Linear layers: the largest need over every
  // row count the context accepts
  for (int m = 1; m <= max_rows; ++m) {
    const int hh = d.hidden, ff = d.ffn;
    c->gpart_bytes = std::max({c->gpart_bytes, linear_workspace_bytes(d.dtype, m, 3 * hh, hh),
                               linear_workspace_bytes(d.dtype, m, hh, hh),
                               linear_workspace_bytes(d.dtype, m, ff, hh),
                               linear_workspace_bytes(d.dtype, m, hh, ff)});
  }
  c->off_gpart = take(c->gpart_bytes);
  c->meta_bytes = sizeof(DevReq) * max_reqs + sizeof(int32_t) * R +
                  sizeof(SplitItem) * c->max_items + sizeof(SplitRow) * R +
                  sizeof(PrefillItem) * c->max_pf + sizeof(PrefillSlot) * c->max_pf * d.heads +
                  16 * 9;
  c->off_meta = take(c->meta_bytes);
  c->ws_bytes = o;
  hipError_t e = hipGetDevice(&c->device);
  for (int i = 0; i < NSLOT && e == hipSuccess; ++i) {
    e = hipHostMalloc(&c->staging[i], c->meta_bytes, hipHostMallocDefault);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&c->ev[i], hipEventDisableTiming);
  }
  if (e != hipSuccess) {
    orca_destroy(c);
    return hip_fail(e, "orca_create");
  }
  *out = c;
  return ORCA_OK;
}

orca_status orca_destroy(orca_ctx* c) {
  if (!c) return ORCA_OK;
  for (hipEvent_t e : c->probe_ev) {
    (void)hipEventSynchronize(e);
    (void)hipEventDestroy(e);
  }
  for (int i = 0; i < NSLOT; ++i) {
    if (c->ev[i]) {
      (void)hipEventSynchronize(c->ev[i]);
      (void)hipEventDestroy(c->ev[i]);
    }
    if (c->staging[i]) (void)hipHostFree(c->staging[i]);
  }
  delete c;
  return ORCA_OK;
}

size_t orca_workspace_bytes(const orca_ctx* c) { return c ? c->ws_bytes : 0; }

static orca_status check_ws(const orca_ctx* c, const void* ws, size_t ws_bytes) {
  ORCA_CHECK_ARG(ws != nullptr, "workspace is NULL");
  ORCA_CHECK_ARG(reinterpret_cast<uintptr_t>(ws) % ALIGN == 0, "workspace not 256-byte aligned");
  ORCA_CHECK_ARG(ws_bytes >= c->ws_bytes, "workspace of %zu bytes, need %zu", ws_bytes,
                 c->ws_bytes);
  return ORCA_OK;
}

static orca_status run_attention(orca_ctx* c, int layer, AttnArgs aa, const void* q, void* o,
                                 hipStream_t s) {
  const size_t pool = c->layer_pool_elems() * dsize(c->desc.dtype);
  aa.q = q;
  aa.o = o;
  aa.kv_pool = static_cast<char*>(c->kv_pool) + pool * layer;
  HIP_TRY(launch_attention(aa, s), "attention launch");
  return ORCA_OK;
}

orca_status orca_iteration(orca_ctx* c, const orca_req_desc* reqs, int32_t n_reqs, const void* x,
                           void* y, void* workspace, size_t ws_bytes, void* stream) {
  clear_error();
  ORCA_CHECK_ARG(c != nullptr, "NULL context");
  orca_status st = check_ws(c, workspace, ws_bytes);
  if (st != ORCA_OK) return st;
  ORCA_CHECK_ARG(n_reqs == 0 || (x && y), "x / y is NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  Plan p;
  AttnArgs aa;
  st = stage(c, reqs, n_reqs, ws, s, p, aa);
  if (st != ORCA_OK || p.rows == 0) return st;

  const orca_model_desc& d = c->desc;
  const int R = p.rows, H = d.hidden, F = d.ffn, dt = d.dtype;
  float* resid = reinterpret_cast<float*>(ws + c->off_resid);
  void* a = ws + c->off_a;
  void* q = ws + c->off_q;
  void* o = ws + c->off_o;
  void* f = ws + c->off_f;
  const int32_t* row_dst = reinterpret_cast<const int32_t*>(ws + c->off_meta + p.off_row_dst);
  const size_t pool = c->layer_pool_elems() * dsize(dt);
  void* gp = ws + c->off_gpart;
  const size_t gpb = c->gpart_bytes;

  const bool probe = c->probe_step >= 0;
  auto mark = [&](int l, int step, int end) -> hipError_t {
    if (!probe || step != c->probe_step) return hipSuccess;
    return hipEventRecord(c->probe_ev[2 * l + end], s);
  };
  auto probe_mid = [&](int l, int step) -> hipEvent_t {
    return probe && step == c->probe_step ? c->probe_ev[2 * l + 1] : nullptr;
  };
  HIP_TRY(launch_to_f32(dt, x, resid, int64_t(R) * H, s), "input conversion");
  // LN1 of layer 0 here; every later LayerNorm runs with the residual
  // Linear before it (one kernel with its split-K reduce when that applies)
  HIP_TRY(launch_layernorm(dt, resid, c->layers[0].ln1_g, c->layers[0].ln1_b, a, R, H, d.ln_eps, s),
          "LN1");
  for (int l = 0; l < d.layers; ++l) {
    const orca_layer_weights& w = c->layers[l];
    QkvDest qd{q, static_cast<char*>(c->kv_pool) + pool * l, row_dst, H, H / d.heads,
               d.kv_capacity};
    HIP_TRY(mark(l, ORCA_STEP_QKV, 0), "timing event");
    HIP_TRY(launch_linear(dt, EPI_QKV, a, w.w_qkv, w.b_qkv, nullptr, &qd, R, 3 * H, H, gp, gpb, s), "QKV");
    HIP_TRY(mark(l, ORCA_STEP_QKV, 1), "timing event");
    HIP_TRY(mark(l, ORCA_STEP_ATTENTION, 0), "timing event");
    st = run_attention(c, l, aa, q, o, s);
    if (st != ORCA_OK) return st;
    HIP_TRY(mark(l, ORCA_STEP_ATTENTION, 1), "timing event");
    HIP_TRY(mark(l, ORCA_STEP_OUT_PROJ, 0), "timing event");
    HIP_TRY(launch_linear_resid_ln(dt, o, w.w_o, w.b_o, resid, R, H, H, gp, gpb, w.ln2_g, w.ln2_b, a,
                                   d.ln_eps, s, probe_mid(l, ORCA_STEP_OUT_PROJ)),
            "output projection + LN2");
    HIP_TRY(mark(l, ORCA_STEP_FFN1, 0), "timing event");
    HIP_TRY(launch_linear(dt, ORCA_EPI_BIAS_GELU, a, w.w_1, w.b_1, f, nullptr, R, F, H, gp, gpb, s), "FFN1");
    HIP_TRY(mark(l, ORCA_STEP_FFN1, 1), "timing event");
    HIP_TRY(mark(l, ORCA_STEP_FFN2, 0), "timing event");
    if (l + 1 < d.layers) {
      const orca_layer_weights& wn = c->layers[l + 1];
      HIP_TRY(launch_linear_resid_ln(dt, f, w.w_2, w.b_2, resid, R, H, F, gp, gpb, wn.ln1_g, wn.ln1_b,
                                     a, d.ln_eps, s, probe_mid(l, ORCA_STEP_FFN2)),
              "FFN2 + next LN1");
    } else {
      HIP_TRY(launch_linear(dt, ORCA_EPI_BIAS_RESID, f, w.w_2, w.b_2, resid, nullptr, R, H, F, gp, gpb,
                            s),
              "FFN2");
      HIP_TRY(mark(l, ORCA_STEP_FFN2, 1), "timing event");
    }
  }
  if (probe) c->probe_recorded = true;
  HIP_TRY(launch_from_f32(dt, resid, y, int64_t(R) * H, s), "output conversion");
  return ORCA_OK;
}

// ------------------------------------------------------------ step timing

orca_status orca_time_step(orca_ctx* c, int32_t step) {
  clear_error();
  ORCA_CHECK_ARG(c != nullptr, "NULL context");
  ORCA_CHECK_ARG(step >= -1 && step <= ORCA_STEP_FFN2, "unknown step %d", step);
  if (step >= 0 && c->probe_ev.empty()) {
    c->probe_ev.assign(2 * size_t(c->desc.layers), nullptr);
    for (hipEvent_t& e : c->probe_ev) {
      const hipError_t r = hipEventCreate(&e);
      if (r != hipSuccess) {
        for (hipEvent_t& f : c->probe_ev)
          if (f) (void)hipEventDestroy(f);
        c->probe_ev.clear();
        return hip_fail(r, "orca_time_step");
      }
    }
  }
  c->probe_step = step;
  c->probe_recorded = false;
  return ORCA_OK;
}

orca_status orca_step_times(orca_ctx* c, float* ms, int32_t n) {
  clear_error();
  ORCA_CHECK_ARG(c != nullptr && (ms != nullptr || n == 0), "NULL argument");
  ORCA_CHECK_ARG(c->probe_step >= 0 && c->probe_recorded,
                 "no iteration has run since a step was chosen for timing");
  const int layers = std::min<int>(n, c->desc.layers);
  HIP_TRY(hipEventSynchronize(c->probe_ev[2 * size_t(c->desc.layers) - 1]), "timing wait");
  for (int l = 0; l < layers; ++l)
    HIP_TRY(hipEventElapsedTime(&ms[l], c->probe_ev[2 * l], c->probe_ev[2 * l + 1]),
            "timing read");
  return ORCA_OK;
}

// ------------------------------------------------------------ single steps

orca_status orca_op_layernorm(int32_t dtype, const float* x, const void* gamma, const void* beta,
                              void* out, int32_t rows, int32_t hidden, float eps, void* stream) {
  clear_error();
  ORCA_CHECK_ARG(dtype == ORCA_F32 || dtype == ORCA_BF16, "unknown dtype %d", dtype);
  ORCA_CHECK_ARG(rows >= 0 && hidden >= 4 && hidden % 4 == 0 && hidden <= 12288,
                 "rows %d hidden %d (hidden must be a multiple of 4, at most 12288)", rows, hidden);
  ORCA_CHECK_ARG(eps > 0.f, "eps must be > 0");
  ORCA_CHECK_ARG(rows == 0 || (x && gamma && beta && out), "NULL argument");
  HIP_TRY(launch_layernorm(dtype, x, gamma, beta, out, rows, hidden, eps,
                           static_cast<hipStream_t>(stream)), "layernorm launch");
  return ORCA_OK;
}

int32_t orca_op_linear_variant(int32_t dtype, int32_t m, int32_t n, int32_t k) {
  if ((dtype != ORCA_BF16 && dtype != ORCA_F32) || m < 1 || n < 64 || k < 64 || n % 64 || k % 64)
    return -2;
  return linear_plan_variant(dtype, m, n, k);
}

int32_t orca_op_prefill_keys(int32_t heads, int32_t tiles) {
  if (heads < 1 || tiles < 0) return -2;
  return prefill_keys_per_step(heads, tiles);
}

int32_t orca_op_prefill_order(const orca_req_desc* reqs, int32_t n, int32_t heads,
                              int32_t* req_out, int32_t* q0_out, int32_t* head_out, int32_t cap) {
  if (n < 0 || heads < 1 || cap < 0 || (n > 0 && !reqs)) return -2;
  std::vector<DevReq> dr(n);
  std::vector<PrefillItem> pf;
  for (int i = 0; i < n; ++i) {
    const orca_req_desc& r = reqs[i];
    if (r.q_len < 0 || r.kv_len < 0) return -2;
    dr[i] = DevReq{r.q_offset, r.q_len, r.kv_len, r.phase, r.kv_base};
    if (r.phase == ORCA_INITIATION)
      for (int q0 = 0; q0 < r.q_len; q0 += PREFILL_ROWS)
        pf.push_back(PrefillItem{i, q0, std::min(r.q_len, q0 + PREFILL_ROWS), 0});
  }
  const int64_t total = int64_t(pf.size()) * heads;
  if (total > INT32_MAX) return -2;
  std::vector<PrefillSlot> slots(total);
  prefill_schedule(dr.data(), n, pf.data(), int(pf.size()), heads, slots.data());
  if (cap > 0 && (!req_out || !q0_out || !head_out)) return -2;
  for (int64_t i = 0; i < std::min<int64_t>(total, cap); ++i) {
    const PrefillItem& t = pf[slots[i].item];
    req_out[i] = t.req;
    q0_out[i] = t.q0;
    head_out[i] = slots[i].head;
  }
  return int32_t(total);
}

size_t orca_op_linear_workspace_bytes(int32_t dtype, int32_t m, int32_t n, int32_t k) {
  if (m < 0 || n < 64 || k < 64 || n % 64 || k % 64) return 0;
  return linear_workspace_bytes(dtype, m, n, k);
}

orca_status orca_op_linear(int32_t dtype, int32_t epilogue, const void* a, const void* w,
                           const void* bias, void* out, int32_t m, int32_t n, int32_t k,
                           void* workspace, size_t ws_bytes, void* stream) {
  clear_error();
  ORCA_CHECK_ARG(dtype == ORCA_F32 || dtype == ORCA_BF16, "unknown dtype %d", dtype);
  ORCA_CHECK_ARG(epilogue >= ORCA_EPI_BIAS && epilogue <= ORCA_EPI_BIAS_RESID,
                 "unknown epilogue %d", epilogue);
  ORCA_CHECK_ARG(m >= 0 && n >= 64 && k >= 64, "shape m %d n %d k %d", m, n, k);
  if (n % 64 || k % 64) {
    set_error("unsupported shape: n %d and k %d must be multiples of 64", n, k);
    return ORCA_ERR_UNSUPPORTED;
  }
  ORCA_CHECK_ARG(m == 0 || (a && w && bias && out), "NULL argument");
  HIP_TRY(launch_linear(dtype, epilogue, a, w, bias, out, nullptr, m, n, k, workspace, ws_bytes,
                        static_cast<hipStream_t>(stream)), "linear launch");
  return ORCA_OK;
}

orca_status orca_op_qkv(int32_t dtype, const void* a, const void* w_qkv, const void* b_qkv,
                        void* q_out, void* kv_pool_l, const int32_t* row_dst,
                        int32_t m, int32_t hidden, int32_t heads, int64_t kv_capacity,
                        void* workspace, size_t ws_bytes, void* stream) {
  clear_error();
  ORCA_CHECK_ARG(dtype == ORCA_F32 || dtype == ORCA_BF16, "unknown dtype %d", dtype);
  ORCA_CHECK_ARG(m >= 0 && hidden >= 64 && heads >= 1 && hidden % heads == 0 && kv_capacity >= 1,
                 "shape m %d hidden %d heads %d capacity %lld", m, hidden, heads,
                 (long long)kv_capacity);
  if (hidden % 64 || !head_dim_ok(dtype, hidden / heads)) {
    set_error("unsupported shape: hidden %d head_dim %d", hidden, hidden / heads);
    return ORCA_ERR_UNSUPPORTED;
  }
  ORCA_CHECK_ARG(m == 0 || (a && w_qkv && b_qkv && q_out && kv_pool_l && row_dst),
                 "NULL argument");
  QkvDest qd{q_out, kv_pool_l, row_dst, hidden, hidden / heads, kv_capacity};
  HIP_TRY(launch_linear(dtype, EPI_QKV, a, w_qkv, b_qkv, nullptr, &qd, m, 3 * hidden, hidden,
                        workspace, ws_bytes,
                        static_cast<hipStream_t>(stream)), "qkv launch");
  return ORCA_OK;
}

orca_status orca_op_attention(orca_ctx* c, int32_t layer, const orca_req_desc* reqs,
                              int32_t n_reqs, const void* q, void* o, void* workspace,
                              size_t ws_bytes, void* stream) {
  clear_error();
  ORCA_CHECK_ARG(c != nullptr, "NULL context");
  ORCA_CHECK_ARG(layer >= 0 && layer < c->desc.layers, "layer %d out of range", layer);
  orca_status st = check_ws(c, workspace, ws_bytes);
  if (st != ORCA_OK) return st;
  ORCA_CHECK_ARG(n_reqs == 0 || (q && o), "q / o is NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  Plan p;
  AttnArgs aa;
  st = stage(c, reqs, n_reqs, static_cast<char*>(workspace), s, p, aa);
  if (st != ORCA_OK || p.rows == 0) return st;
  return run_attention(c, layer, aa, q, o, s);
}

}  // extern "C"
