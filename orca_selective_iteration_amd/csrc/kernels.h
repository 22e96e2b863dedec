// Host-side launchers of the gfx950 kernels (defined next to each kernel).
// Every launcher enqueues on `stream`, assumes its arguments were validated
// by the caller, and returns the hipError_t of the launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace orca {

// ---- LayerNorm and conversions (ln.hip) ----------------------------------
hipError_t launch_layernorm(int dtype, const float* x, const void* g, const void* b, void* out,
                            int rows, int hidden, float eps, hipStream_t s);
// bf16 only: resid[r] += sum of the `splits` fp32 planes part[s][r] + bias,
// then out[r] = LN(resid[r]); hipErrorNotSupported past hidden = 12288
hipError_t launch_reduce_resid_ln(const float* part, int splits, const void* bias, float* resid,
                                  int rows, int hidden, const void* g, const void* b, void* out,
                                  float eps, hipStream_t s);
hipError_t launch_to_f32(int dtype, const void* in, float* out, int64_t n, hipStream_t s);
hipError_t launch_from_f32(int dtype, const float* in, void* out, int64_t n, hipStream_t s);

// ---- Linear layers (gemm.hip) ---------------------------------------------
struct QkvDest {
  void* q_out;          // [m][H]
  void* kv_pool;        // one layer: [heads][cap][2][d] (key row, then value row)
  const int32_t* row_dst;
  int hidden, head_dim;
  int64_t cap;
};
// epilogue: ORCA_EPI_* or EPI_QKV (3).  For EPI_QKV, `out` is ignored and
// `qkv` describes the destinations.
constexpr int EPI_QKV = 3;
// internal: fp32 partial sums of a K split, no bias (the few-rows path)
constexpr int EPI_PARTIAL = 4;
// bf16 problems whose tiles are too few to fill the GPU (on 32/64/128-row
// tiles at most half a round of resident workgroups, at any row count; 256
// x 256 tiles short of one round when splitting K fills whole rounds
// better) take a split-K path when `ws` holds
// linear_workspace_bytes(dtype, m, n, k) bytes (fp32 partial sums);
// otherwise, and for every other shape, the tiled kernels run and `ws` is
// not touched.  The half-round test bounds the partial sums: tiles x splits
// stays within one round, so splits * m * n <= 512 * 128 * 128 elements.
constexpr int SPLIT_MAX_SPLITS = 16;
size_t linear_workspace_bytes(int dtype, int m, int n, int k);
// The tile variant a bf16 launch of this problem takes (ORCA_GEMM_VARIANT
// honoured, fallbacks applied; 10 is split-K given its workspace); -1 for
// fp32.
int linear_plan_variant(int dtype, int m, int n, int k);
hipError_t launch_linear(int dtype, int epilogue, const void* a, const void* w, const void* bias,
                         void* out, const QkvDest* qkv, int m, int n, int k, void* ws,
                         size_t ws_bytes, hipStream_t s);
// The residual-epilogue Linear (out is the fp32 residual [m][n]) followed
// by the LayerNorm of the new residual into ln_out; on the split-K path the
// two share one kernel after the partial GEMM.  `after_gemm`, when not
// NULL, is recorded on `s` after the GEMM's launches and before the rest.
hipError_t launch_linear_resid_ln(int dtype, const void* a, const void* w, const void* bias,
                                  float* resid, int m, int n, int k, void* ws, size_t ws_bytes,
                                  const void* ln_g, const void* ln_b, void* ln_out, float eps,
                                  hipStream_t s, hipEvent_t after_gemm = nullptr);

// ---- Attention (attn.hip) --------------------------------------------------
// Device request record: same layout as orca_req_desc.
struct DevReq {
  int32_t q_offset, q_len, kv_len, phase;
  int64_t kv_base;
};
// Split-KV work item: query row `row` of request `req`, keys [c0, c1).
struct SplitItem {
  int32_t row, req, c0, c1;
};
// Query rows served by the split-KV path, with their item range.
struct SplitRow {
  int32_t row, item_begin, item_count, req;
};
// Prefill (initiation) tile: request `req`, query rows [q0, q1) of its prompt.
struct PrefillItem {
  int32_t req, q0, q1, pad;
};
// One workgroup of a prefill launch: tile `item` (an index into the prefill
// items) for head `head`.
struct PrefillSlot {
  int32_t item, head;
};

struct AttnArgs {
  int dtype, hidden, heads, head_dim;
  int64_t cap;
  const void* q;          // [rows][H]
  void* o;                // [rows][H]
  const void* kv_pool;    // one layer: [heads][cap][2][d] (key row, then value row)
  const DevReq* reqs;
  const SplitItem* items;  int n_items;
  const SplitRow* srows;   int n_srows;
  const PrefillItem* pf;   int n_pf;
  const PrefillSlot* pf_slots;   // [n_pf * heads]: what workgroup i computes
  float* part_o;          // [n_items][heads][d]
  float* part_ml;         // [n_items][heads][2]
};

// Keys per split-KV work item for increment rows.
constexpr int SPLIT_CHUNK = 512;
// Query positions per prefill (initiation) workgroup.
constexpr int PREFILL_ROWS = 128;

hipError_t launch_attention(const AttnArgs& a, hipStream_t s);
// Keys per step of the prefill form a launch of `n_pf` tiles over `heads`
// heads takes (64: two workgroups per CU; 32: three); ORCA_PF_KEYS pins it.
int prefill_keys_per_step(int heads, int n_pf);
// Order of a prefill launch's workgroups: false, the tiles longest-first
// with the heads of one tile adjacent; true, grouped by (request, head) per
// XCD (prefill_schedule); ORCA_PF_ORDER (0 or 1) pins it.
bool prefill_grouped(int heads, int n_pf);
// Fills slots[0 .. n_pf * heads) for the prefill tiles pf[0 .. n_pf) of
// requests reqs, sorting pf longest-first (by cached prefix + last query).
void prefill_schedule(const DevReq* reqs, int n_reqs, PrefillItem* pf, int n_pf, int heads,
                      PrefillSlot* slots);

}  // namespace orca
