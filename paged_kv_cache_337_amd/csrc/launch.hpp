// Host-side launch entry points of the device kernels (internal, not ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

struct PoolGeom {
  void* base;           // device pool buffer
  int32_t L, N, bs, H, D, dtype;
  int32_t elem_bytes;
  size_t layer_elems() const { return static_cast<size_t>(N) * H * 2 * bs * D; }
};

struct DecodeParams {
  const void* pool;          // device pool base
  size_t layer_off;          // element offset of the layer
  int32_t N, H, bs;
  const void* q;             // [S, Hq, D]
  void* out;                 // [S, Hq, D]
  const int32_t* tables;     // [S, max_blocks]
  int32_t max_blocks;
  const int32_t* ctx;        // [S]
  int32_t S, Hq, G;
  int32_t ctx_cap;           // min(max_context_len, max_blocks * bs)
  float scale_log2;          // scale * log2(e)
  int32_t P;                 // partition tokens (the minimum when automatic)
  int32_t auto_partition;    // 1: the plan kernel may raise P (header[2])
  int32_t grid;              // workgroups of the decode kernel
  int32_t first_taken;       // work indices handed out by workgroup id before the counter
  int32_t group;             // partitions per work item: 1, or one per wave (each wave then
                             //    computes one partition and writes its state itself)
  int32_t direct;            // 1: one (sequence, kv head) per workgroup, no plan, no counter
                             //    (every context within one partition, S * H <= grid)
  int32_t max_parts;         // ceil(ctx_cap / P)
  int32_t ws_stride;         // partition-state slots per (sequence, query head) row: max_parts + 1
  int32_t* header;           // [0] work items, [1] next work index, [2] P used, [3] shared groups (device)
  int4* items;               // [S * ws_stride] work items, longest first; records:
                             //   (sequence, partition, context, partitions) without sharing,
                             //   (sequence or ~group, partition slot, first token, end token) with it
  float* ws_o;               // [S, Hq, ws_stride, D]
  float* ws_ml;              // [S, Hq, ws_stride, 2] (max in log2 units, sum)
  int32_t share;             // 1: the plan groups sequences whose tables share leading blocks
  int32_t share_nmax;        // sequences per shared work item (their G query heads each: <= 16 columns)
  int32_t* seq_np;           // [S] partition states of each sequence (sharing mode)
  int4* groups;              // [S / 2] member sequences of each shared group (-1 = none)
  const int32_t* host_plan;  // sharing groups found on the host (pa_batch_share_plan's words), or NULL
  int32_t flat;              // 1: no block table; tables[i] (max_blocks = 1) is sequence i's first
                             //    block and its blocks are consecutive (contiguous-layout comparison)
  // new tokens written before the decode (pa_decode_step; w_tokens = 0: none)
  const void* w_k;           // [w_tokens, H, D] pool dtype
  const void* w_v;
  const int32_t* w_slots;    // [w_tokens] global slots, -1 = skip
  int32_t w_tokens;
};

struct PrefillParams {
  const void* pool;            // device pool base
  size_t layer_off;            // element offset of the layer
  int32_t N, H, bs;
  const void* q;               // [num_q_tokens, Hq, D]
  void* out;                   // [num_q_tokens, Hq, D]
  const int32_t* query_start;  // [S + 1] offsets of each sequence's new tokens
  int32_t num_q_tokens;        // rows of q and out
  int32_t max_query_len;       // bound on new tokens per sequence (sizes the grid)
  const int32_t* tables;       // [S, max_blocks]
  int32_t max_blocks;
  const int32_t* ctx;          // [S] context lengths, new tokens included
  int32_t S, Hq, G;
  int32_t ctx_cap;             // min(max_context_len, max_blocks * bs)
  float scale_log2;            // scale * log2(e)
  int32_t tiles;               // row tiles per (sequence, kv head) in the grid (set at launch)
  int32_t lpt;                 // 1: heaviest-first workgroup order (set at launch)
};

// Workspace of pa_decode: a small header, the work-item list, the sharing
// plan's per-sequence partition counts and groups, and (only when some
// context spans several partitions) the float32 partition states.
// With several partitions per context, every (sequence, query head) row has
// ws_stride = max_parts + 1 state slots: splitting a context at the end of a
// prefix it shares with other sequences can add one partition.
struct WsLayout {
  size_t header_off, items_off, np_off, groups_off, o_off, ml_off, total;
  int stride;
};

inline WsLayout decode_ws_layout(int S, int Hq, int max_parts, int D) {
  auto align = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  WsLayout w;
  w.stride = max_parts > 1 ? max_parts + 1 : 1;
  w.header_off = 0;
  w.items_off = 256;
  w.np_off = align(w.items_off + static_cast<size_t>(S) * w.stride * sizeof(int4));
  w.groups_off = align(w.np_off + static_cast<size_t>(S) * sizeof(int32_t));
  w.o_off = align(w.groups_off + static_cast<size_t>(S / 2 + 1) * sizeof(int4));
  const size_t parts = max_parts > 1 ? static_cast<size_t>(S) * Hq * w.stride : 0;
  w.ml_off = align(w.o_off + parts * D * sizeof(float));
  w.total = align(w.ml_off + parts * 2 * sizeof(float));
  return w;
}

// The write kernel over layer `layer`, or (layer_byte_off >= 0) over the
// layer that starts layer_byte_off bytes into the pool.
hipError_t launch_write_kv(const PoolGeom& g, int layer, const void* k, const void* v,
                           const int32_t* slots, int num_tokens, hipStream_t stream, int64_t layer_byte_off = -1);

hipError_t launch_copy_blocks(const PoolGeom& g, const int32_t* pairs, int n, hipStream_t stream);

// Whole-block copies between the pool and a host tier (host: device-usable
// address of pinned host memory holding host_blocks blocks of every layer).
hipError_t launch_swap_blocks(const PoolGeom& g, const int32_t* pairs, int n, void* host, int64_t host_blocks,
                              int dir, hipStream_t stream);

// Returns hipErrorInvalidValue when no kernel variant covers (dtype, D, G).
hipError_t launch_decode(const DecodeParams& p, int dtype, int D, hipStream_t stream);

bool decode_supported(int dtype, int D, int G);

// Read probe: n chunks of 8 KiB of buf in the order of ids (device), with one
// of the probe's load forms, wg_per_cu workgroups of four waves per CU and
// in_flight chunks in flight per wave.
bool probe_supported(int load_form, int wg_per_cu, int in_flight);
hipError_t launch_probe_read(const void* buf, int64_t nchunks_buf, const int32_t* ids, int n, int load_form,
                             int wg_per_cu, int in_flight, void* sink, hipStream_t stream);

// Causal prefill of the newest tokens of each sequence (same shape support as
// decode).  Returns hipErrorInvalidValue when the grid would exceed its limit.
hipError_t launch_prefill(const PrefillParams& p, int dtype, int D, hipStream_t stream);

// Largest max_query_len a prefill launch accepts for group size G.
int64_t prefill_max_query_len(int G);

}  // namespace pa
