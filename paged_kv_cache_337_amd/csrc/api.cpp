// C ABI of the paged decode library (declared in include/pa.h): argument
// validation, error reporting, the host block manager, and kernel launches.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <exception>
#include <new>
#include <string>
#include <unordered_map>
#include <vector>

#include "allocator.hpp"
#include "api_internal.hpp"
#include "launch.hpp"
#include "pa.h"

struct pa_pool {
  pa_pool_desc desc;
  void* buf;
  size_t bytes;
  pa::BlockAllocator alloc;
  pa_pool(const pa_pool_desc& d, void* b, size_t n)
      : desc(d), buf(b), bytes(n), alloc(d.num_blocks, d.block_size) {}
};

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

int elem_bytes(int32_t dtype) { return dtype == PA_F32 ? 4 : (dtype == PA_F16 || dtype == PA_BF16) ? 2 : 0; }

// Validates a descriptor; returns PA_OK or an error code (message set).
int check_desc(const pa_pool_desc* d) {
  if (!d) return fail(PA_ERR_INVALID_ARG, "descriptor is NULL");
  if (d->num_layers < 0 || d->num_blocks < 0 || d->num_kv_heads < 0 || d->head_dim < 0)
    return fail(PA_ERR_INVALID_ARG, "counts cannot be negative");
  if (d->block_size <= 0) return fail(PA_ERR_INVALID_ARG, "block size must be positive");
  if (d->num_layers == 0 || d->num_kv_heads == 0 || d->head_dim == 0)
    return fail(PA_ERR_INVALID_ARG, "layers, kv heads and head_dim must be positive");
  if (elem_bytes(d->dtype) == 0) return fail(PA_ERR_UNSUPPORTED, "unknown dtype");
  if (d->block_size % 16 || d->block_size > 256)
    return fail(PA_ERR_UNSUPPORTED, "block_size must be a multiple of 16, at most 256");
  if (d->head_dim != 64 && d->head_dim != 128) return fail(PA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (static_cast<int64_t>(d->num_blocks) * d->block_size >= (int64_t{1} << 31))
    return fail(PA_ERR_INVALID_ARG, "num_blocks * block_size must stay below 2^31 slots");
  return PA_OK;
}

size_t required_bytes(const pa_pool_desc& d) {
  // 2 * L * T * H_KV * D * B with T = N * bs.
  return size_t{2} * static_cast<size_t>(d.num_layers) * static_cast<size_t>(d.num_blocks) *
         static_cast<size_t>(d.block_size) * static_cast<size_t>(d.num_kv_heads) *
         static_cast<size_t>(d.head_dim) * static_cast<size_t>(elem_bytes(d.dtype));
}

pa::PoolGeom geom_of(const pa_pool* p) {
  pa::PoolGeom g;
  g.base = p->buf;
  g.L = p->desc.num_layers;
  g.N = p->desc.num_blocks;
  g.bs = p->desc.block_size;
  g.H = p->desc.num_kv_heads;
  g.D = p->desc.head_dim;
  g.dtype = p->desc.dtype;
  g.elem_bytes = elem_bytes(p->desc.dtype);
  return g;
}

// Read on every call (a getenv is far cheaper than any launch), so a process
// can switch validation on and off.
bool debug_enabled() {
  const char* s = std::getenv("PA_DEBUG");
  return s && *s && std::strcmp(s, "0") != 0;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int hip_fail(hipError_t e, const char* what) {
  return fail(PA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

int auto_partition(int bs) {
  // 512 tokens rounded to whole blocks.
  int p = (512 / bs) * bs;
  return p > 0 ? p : bs;
}

template <typename F>
int guarded(F&& f) {
  try {
    return f();
  } catch (const std::bad_alloc&) {
    return fail(PA_ERR_INVALID_ARG, "host allocation failed");
  } catch (const std::exception& e) {
    return fail(PA_ERR_INVALID_ARG, e.what());
  } catch (...) {
    return fail(PA_ERR_INVALID_ARG, "unknown error");
  }
}

// PA_DEBUG check of a write's slot mapping: copied to the host (synchronising
// the stream), every slot in range or -1, no slot twice.
int check_slots_debug(const pa_pool* pool, const int32_t* slot_mapping, int num_tokens, hipStream_t s) {
  std::vector<int32_t> h(num_tokens);
  hipError_t e = hipMemcpyAsync(h.data(), slot_mapping, sizeof(int32_t) * num_tokens, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "PA_DEBUG slot readback");
  const int64_t nslots = static_cast<int64_t>(pool->desc.num_blocks) * pool->desc.block_size;
  std::vector<int32_t> sorted;
  for (int32_t x : h) {
    if (x < -1 || x >= nslots) return fail(PA_ERR_INVALID_ARG, "slot " + std::to_string(x) + " out of range");
    if (x >= 0) sorted.push_back(x);
  }
  std::sort(sorted.begin(), sorted.end());
  if (std::adjacent_find(sorted.begin(), sorted.end()) != sorted.end())
    return fail(PA_ERR_INVALID_ARG, "slot_mapping holds a repeated slot");
  return PA_OK;
}

int alloc_status(pa::AllocResult r, const std::string& msg) {
  switch (r) {
    case pa::AllocResult::Ok:
      return PA_OK;
    case pa::AllocResult::OutOfBlocks:
      return fail(PA_ERR_OUT_OF_BLOCKS, msg);
    default:
      return fail(PA_ERR_INVALID_ARG, msg);
  }
}

}  // namespace

extern "C" {

const char* pa_version(void) { return "pagedattn-mi355x 0.1.0 (gfx950)"; }

const char* pa_last_error(void) { return g_err.c_str(); }

size_t pa_pool_required_bytes(const pa_pool_desc* desc) {
  if (check_desc(desc) != PA_OK) return 0;
  return required_bytes(*desc);
}

int pa_alloc_pool(const pa_pool_desc* desc, void* dev_buf, size_t buf_bytes,
                  const int32_t* free_order, pa_pool** out) {
  return guarded([&]() -> int {
    if (!out) return fail(PA_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    int rc = check_desc(desc);
    if (rc != PA_OK) return rc;
    if (!dev_buf) return fail(PA_ERR_INVALID_ARG, "device buffer is NULL");
    if (reinterpret_cast<uintptr_t>(dev_buf) & 255u)
      return fail(PA_ERR_INVALID_ARG, "device buffer must be 256-byte aligned");
    const size_t need = required_bytes(*desc);
    if (buf_bytes < need)
      return fail(PA_ERR_BUFFER_TOO_SMALL, "buffer holds " + std::to_string(buf_bytes) + " bytes, pool needs " +
                                               std::to_string(need));
    pa_pool* p = new pa_pool(*desc, dev_buf, buf_bytes);
    if (free_order) {
      std::string err;
      if (!p->alloc.set_free_order(free_order, desc->num_blocks, &err)) {
        delete p;
        return fail(PA_ERR_INVALID_ARG, err);
      }
    }
    *out = p;
    return PA_OK;
  });
}

int pa_free(pa_pool* pool) {
  delete pool;
  return PA_OK;
}

int pa_write_kv(pa_pool* pool, int layer, const void* k, const void* v,
                const int32_t* slot_mapping, int num_tokens, void* stream) {
  return guarded([&]() -> int {
    if (!pool) return fail(PA_ERR_INVALID_ARG, "pool is NULL");
    if (layer < 0 || layer >= pool->desc.num_layers) return fail(PA_ERR_INVALID_ARG, "layer out of range");
    if (num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "token count cannot be negative");
    if (num_tokens == 0) return PA_OK;
    if (!k || !v || !slot_mapping) return fail(PA_ERR_INVALID_ARG, "NULL device pointer");
    if (!aligned16(k) || !aligned16(v)) return fail(PA_ERR_INVALID_ARG, "k and v must be 16-byte aligned");
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (debug_enabled()) {
      const int rc = check_slots_debug(pool, slot_mapping, num_tokens, s);
      if (rc != PA_OK) return rc;
    }
    hipError_t e = pa::launch_write_kv(geom_of(pool), layer, k, v, slot_mapping, num_tokens, s);
    return e == hipSuccess ? PA_OK : hip_fail(e, "write_kv launch");
  });
}

size_t pa_decode_workspace_bytes(const pa_pool* pool, int num_seqs, int num_q_heads,
                                 int max_context_len, int partition_tokens) {
  if (!pool || num_seqs <= 0 || num_q_heads <= 0 || max_context_len <= 0) return 0;
  const int P = partition_tokens > 0 ? partition_tokens : auto_partition(pool->desc.block_size);
  const int64_t parts = (static_cast<int64_t>(max_context_len) + P - 1) / P;
  return pa::decode_ws_layout(num_seqs, num_q_heads, static_cast<int>(parts), pool->desc.head_dim).total;
}

int pa_decode(const pa_pool* pool, int layer, const void* q, int num_seqs, int num_q_heads,
              const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
              int max_context_len, float scale, int partition_tokens, void* workspace,
              size_t ws_bytes, void* out, void* stream) {
  return pa::decode_call(pool, layer, q, num_seqs, num_q_heads, block_tables, max_blocks_per_seq, context_lens,
                         max_context_len, scale, partition_tokens, workspace, ws_bytes, out, stream, false);
}

}  // extern "C"

int pa::set_error(int code, const std::string& msg) { return fail(code, msg); }

int pa::decode_call(const pa_pool* pool, int layer, const void* q, int num_seqs, int num_q_heads,
                    const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
                    int max_context_len, float scale, int partition_tokens, void* workspace, size_t ws_bytes,
                    void* out, void* stream, bool noalloc, bool flat, const NewTokens* write,
                    const int32_t* share_plan) {
  return guarded([&]() -> int {
    if (flat) max_blocks_per_seq = 1;
    if (write && write->num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "token count cannot be negative");
    if (write && write->num_tokens > 0) {
      if (!write->k || !write->v || !write->slot_mapping) return fail(PA_ERR_INVALID_ARG, "NULL device pointer");
      if (!aligned16(write->k) || !aligned16(write->v))
        return fail(PA_ERR_INVALID_ARG, "k and v must be 16-byte aligned");
      if (pool && pool->desc.num_kv_heads > 65535) return fail(PA_ERR_UNSUPPORTED, "at most 65535 kv heads");
    }
    if (!pool) return fail(PA_ERR_INVALID_ARG, "pool is NULL");
    const pa_pool_desc& d = pool->desc;
    if (layer < 0 || layer >= d.num_layers) return fail(PA_ERR_INVALID_ARG, "layer out of range");
    if (num_seqs < 0) return fail(PA_ERR_INVALID_ARG, "num_seqs cannot be negative");
    if (num_seqs == 0) return PA_OK;
    if (num_seqs > 65535) return fail(PA_ERR_UNSUPPORTED, "at most 65535 sequences per call");
    if (num_q_heads <= 0 || num_q_heads % d.num_kv_heads)
      return fail(PA_ERR_INVALID_ARG, "num_q_heads must be a positive multiple of num_kv_heads");
    const int G = num_q_heads / d.num_kv_heads;
    if (!pa::decode_supported(d.dtype, d.head_dim, G))
      return fail(PA_ERR_UNSUPPORTED, "no kernel for G=" + std::to_string(G));
    if (!q || !out || !block_tables || !context_lens) return fail(PA_ERR_INVALID_ARG, "NULL device pointer");
    if (!aligned16(q) || !aligned16(out)) return fail(PA_ERR_INVALID_ARG, "q and out must be 16-byte aligned");
    if (max_blocks_per_seq <= 0 || max_context_len <= 0)
      return fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq and max_context_len must be positive");
    if (!std::isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "scale must be finite");
    const int bs = d.block_size;
    int P = partition_tokens;
    const bool automatic = P == 0;
    if (automatic) P = auto_partition(bs);
    if (P < 0 || P % bs || P % 16) return fail(PA_ERR_INVALID_ARG, "partition_tokens must be a multiple of block_size");
    // a flat sequence is bounded by the pool, a paged one by its table row
    const int64_t cap64 = std::min<int64_t>(
        max_context_len, static_cast<int64_t>(flat ? d.num_blocks : max_blocks_per_seq) * bs);
    const int ctx_cap = static_cast<int>(cap64);
    const int max_parts = static_cast<int>((cap64 + P - 1) / P);
    const pa::WsLayout wl = pa::decode_ws_layout(num_seqs, num_q_heads, max_parts, d.head_dim);
    if (noalloc && wl.total > ws_bytes)
      return fail(PA_ERR_BUFFER_TOO_SMALL, "this decode needs " + std::to_string(wl.total) +
                                               " bytes of scratch; the static scratch of pa_decode_noalloc holds " +
                                               std::to_string(ws_bytes) + " (use pa_decode with a caller workspace)");
    if (!workspace || ws_bytes < wl.total)
      return fail(PA_ERR_BUFFER_TOO_SMALL, "workspace needs " + std::to_string(wl.total) + " bytes");
    if (reinterpret_cast<uintptr_t>(workspace) & 255u)
      return fail(PA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (!noalloc && debug_enabled() && write && write->num_tokens > 0) {
      const int rc = check_slots_debug(pool, write->slot_mapping, write->num_tokens, s);
      if (rc != PA_OK) return rc;
    }
    if (!noalloc && debug_enabled()) {
      std::vector<int32_t> hc(num_seqs), ht(static_cast<size_t>(num_seqs) * max_blocks_per_seq);
      hipError_t e = hipMemcpyAsync(hc.data(), context_lens, sizeof(int32_t) * num_seqs, hipMemcpyDeviceToHost, s);
      if (e == hipSuccess)
        e = hipMemcpyAsync(ht.data(), block_tables, sizeof(int32_t) * ht.size(), hipMemcpyDeviceToHost, s);
      if (e == hipSuccess) e = hipStreamSynchronize(s);
      if (e != hipSuccess) return hip_fail(e, "PA_DEBUG readback");
      for (int i = 0; i < num_seqs; ++i) {
        if (hc[i] < 1 || hc[i] > ctx_cap)
          return fail(PA_ERR_INVALID_ARG, "context_lens[" + std::to_string(i) + "] out of range");
        const int nb = (hc[i] + bs - 1) / bs;
        if (flat) {
          if (ht[i] < 0 || static_cast<int64_t>(ht[i]) + nb > d.num_blocks)
            return fail(PA_ERR_INVALID_ARG, "first_block[" + std::to_string(i) + "] range beyond the pool");
          continue;
        }
        for (int b = 0; b < nb; ++b) {
          const int32_t id = ht[static_cast<size_t>(i) * max_blocks_per_seq + b];
          if (id < 0 || id >= d.num_blocks)
            return fail(PA_ERR_INVALID_ARG, "block_tables[" + std::to_string(i) + "][" + std::to_string(b) + "] invalid");
        }
      }
    }
    pa::DecodeParams p{};
    p.pool = pool->buf;
    p.layer_off = static_cast<size_t>(layer) * d.num_blocks * d.num_kv_heads * 2 * static_cast<size_t>(bs) * d.head_dim;
    p.N = d.num_blocks;
    p.H = d.num_kv_heads;
    p.bs = bs;
    p.q = q;
    p.out = out;
    p.tables = block_tables;
    p.max_blocks = max_blocks_per_seq;
    p.ctx = context_lens;
    p.S = num_seqs;
    p.Hq = num_q_heads;
    p.G = G;
    p.ctx_cap = ctx_cap;
    p.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
    p.P = P;
    p.auto_partition = automatic ? 1 : 0;
    p.max_parts = max_parts;
    p.ws_stride = wl.stride;
    char* ws = static_cast<char*>(workspace);
    p.header = reinterpret_cast<int32_t*>(ws + wl.header_off);
    p.items = reinterpret_cast<int4*>(ws + wl.items_off);
    p.seq_np = reinterpret_cast<int32_t*>(ws + wl.np_off);
    p.groups = reinterpret_cast<int4*>(ws + wl.groups_off);
    p.ws_o = max_parts > 1 ? reinterpret_cast<float*>(ws + wl.o_off) : nullptr;
    p.ws_ml = max_parts > 1 ? reinterpret_cast<float*>(ws + wl.ml_off) : nullptr;
    // Sequences can share blocks only if the block manager holds a block
    // with more than one reference (forked branches, cached prefixes).  Then
    // the plan looks for sequences of this batch whose tables begin with the
    // same blocks and reads each such common prefix once for all of them;
    // otherwise it keeps the plain plan.  The plan itself verifies every
    // shared block id, so tables from any source stay correct either way.
    p.share = !flat && pool->alloc.shared_blocks() > 0 ? 1 : 0;
    p.host_plan = p.share ? share_plan : nullptr;
    p.flat = flat ? 1 : 0;
    if (write && write->num_tokens > 0) {
      p.w_k = write->k;
      p.w_v = write->v;
      p.w_slots = write->slot_mapping;
      p.w_tokens = write->num_tokens;
    }
    hipError_t e = pa::launch_decode(p, d.dtype, d.head_dim, s);
    return e == hipSuccess ? PA_OK : hip_fail(e, "decode launch");
  });
}

extern "C" {

int pa_decode_step(pa_pool* pool, int layer, const void* k, const void* v, const int32_t* slot_mapping,
                   int num_tokens, const void* q, int num_seqs, int num_q_heads, const int32_t* block_tables,
                   int max_blocks_per_seq, const int32_t* context_lens, int max_context_len, float scale,
                   int partition_tokens, void* workspace, size_t ws_bytes, void* out, void* stream) {
  const pa::NewTokens w{k, v, slot_mapping, num_tokens};
  if (num_seqs == 0 && num_tokens > 0)  // nothing to decode: the write alone
    return pa_write_kv(pool, layer, k, v, slot_mapping, num_tokens, stream);
  return pa::decode_call(pool, layer, q, num_seqs, num_q_heads, block_tables, max_blocks_per_seq, context_lens,
                         max_context_len, scale, partition_tokens, workspace, ws_bytes, out, stream, false, false,
                         &w);
}

int pa_decode_step_shared(pa_pool* pool, int layer, const void* k, const void* v, const int32_t* slot_mapping,
                          int num_tokens, const void* q, int num_seqs, int num_q_heads,
                          const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
                          int max_context_len, float scale, int partition_tokens, void* workspace,
                          size_t ws_bytes, void* out, void* stream, const int32_t* share_plan) {
  const pa::NewTokens w{k, v, slot_mapping, num_tokens};
  if (num_seqs == 0 && num_tokens > 0)
    return pa_write_kv(pool, layer, k, v, slot_mapping, num_tokens, stream);
  return pa::decode_call(pool, layer, q, num_seqs, num_q_heads, block_tables, max_blocks_per_seq, context_lens,
                         max_context_len, scale, partition_tokens, workspace, ws_bytes, out, stream, false, false,
                         &w, share_plan);
}

size_t pa_share_plan_words(int num_seqs) {
  if (num_seqs < 0) return 0;
  return 3 + 2 * static_cast<size_t>(num_seqs) + 4 * (static_cast<size_t>(num_seqs) / 2 + 1);
}

int pa_batch_share_plan(const pa_pool* pool, const int* seqs, int num_seqs, int num_q_heads, int32_t* plan_out) {
  return guarded([&]() -> int {
    if (!pool || !plan_out || (num_seqs > 0 && !seqs)) return fail(PA_ERR_INVALID_ARG, "NULL argument");
    if (num_seqs < 0) return fail(PA_ERR_INVALID_ARG, "num_seqs cannot be negative");
    const pa_pool_desc& d = pool->desc;
    if (num_q_heads <= 0 || num_q_heads % d.num_kv_heads)
      return fail(PA_ERR_INVALID_ARG, "num_q_heads must be a positive multiple of num_kv_heads");
    for (int i = 0; i < num_seqs; ++i) {
      if (!pool->alloc.live(seqs[i])) return fail(PA_ERR_INVALID_ARG, "unknown or released sequence");
      if (pool->alloc.swapped(seqs[i])) return fail(PA_ERR_INVALID_ARG, "sequence is swapped out");
    }
    const int S = num_seqs, bs = d.block_size, G = num_q_heads / d.num_kv_heads;
    const int nmax = std::min(4, 16 / G);
    int32_t* sub = plan_out + 3;
    int32_t* shared = plan_out + 3 + S;
    int32_t* members = plan_out + 3 + 2 * static_cast<size_t>(S);
    std::fill(plan_out, plan_out + pa_share_plan_words(S), 0);
    plan_out[1] = S;
    plan_out[2] = nmax;
    std::fill(sub, sub + S, -1);
    std::fill(members, members + 4 * (static_cast<size_t>(S) / 2 + 1), -1);
    // groups: rows whose first full block is the same block, in batch order
    std::vector<int> nfb(S);
    std::unordered_map<int32_t, std::vector<int>> group_of;
    std::vector<int32_t> firsts;
    for (int i = 0; i < S; ++i) {
      const auto& t = pool->alloc.table(seqs[i]);
      nfb[i] = pool->alloc.length(seqs[i]) / bs;
      if (nfb[i] > 0 && !t.empty() && t[0] >= 0 && t[0] < d.num_blocks) {
        auto it = group_of.find(t[0]);
        if (it == group_of.end()) {
          firsts.push_back(t[0]);
          group_of.emplace(t[0], std::vector<int>{i});
        } else {
          it->second.push_back(i);
        }
      }
    }
    // groups in the order of their leaders (lowest rows), as on the device
    std::sort(firsts.begin(), firsts.end(),
              [&](int32_t a, int32_t b) { return group_of[a][0] < group_of[b][0]; });
    int K = 0;
    if (nmax >= 2) {
      for (int32_t f : firsts) {
        const std::vector<int>& mem = group_of[f];
        const int gn = static_cast<int>(mem.size());
        if (gn < 2) continue;
        const auto& lead = pool->alloc.table(seqs[mem[0]]);
        const int gsub = gn / nmax + (gn % nmax >= 2 ? 1 : 0);
        for (int sg = 0; sg < gsub; ++sg) {
          int common = INT32_MAX;
          const int r0 = sg * nmax, r1 = std::min(r0 + nmax, gn);
          for (int r = r0; r < r1; ++r) {
            const int i = mem[r];
            int c = nfb[i];
            if (r > 0) {
              const auto& t = pool->alloc.table(seqs[i]);
              const int cap = std::min(nfb[i], nfb[mem[0]]);
              c = 0;
              while (c < cap && t[c] == lead[c]) ++c;
            }
            common = std::min(common, c);
          }
          if (static_cast<int64_t>(common) * bs < 256) continue;
          for (int r = r0; r < r1; ++r) {
            sub[mem[r]] = K;
            shared[mem[r]] = common * bs;
            members[4 * static_cast<size_t>(K) + (r - r0)] = mem[r];
          }
          ++K;
        }
      }
    }
    plan_out[0] = K;
    return PA_OK;
  });
}

int pa_decode_contiguous(const pa_pool* pool, int layer, const void* q, int num_seqs, int num_q_heads,
                         const int32_t* first_block, const int32_t* context_lens, int max_context_len,
                         float scale, int partition_tokens, void* workspace, size_t ws_bytes, void* out,
                         void* stream) {
  return pa::decode_call(pool, layer, q, num_seqs, num_q_heads, first_block, 1, context_lens, max_context_len,
                         scale, partition_tokens, workspace, ws_bytes, out, stream, false, true);
}

int pa_prefill(const pa_pool* pool, int layer, const void* q, int num_seqs, int num_q_heads,
               const int32_t* query_start, int num_query_tokens, int max_query_len,
               const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
               int max_context_len, float scale, void* out, void* stream) {
  return guarded([&]() -> int {
    if (!pool) return fail(PA_ERR_INVALID_ARG, "pool is NULL");
    const pa_pool_desc& d = pool->desc;
    if (layer < 0 || layer >= d.num_layers) return fail(PA_ERR_INVALID_ARG, "layer out of range");
    if (num_seqs < 0 || num_query_tokens < 0 || max_query_len < 0)
      return fail(PA_ERR_INVALID_ARG, "counts cannot be negative");
    if (num_seqs == 0 || num_query_tokens == 0) return PA_OK;
    if (num_q_heads <= 0 || num_q_heads % d.num_kv_heads)
      return fail(PA_ERR_INVALID_ARG, "num_q_heads must be a positive multiple of num_kv_heads");
    const int G = num_q_heads / d.num_kv_heads;
    if (!pa::decode_supported(d.dtype, d.head_dim, G))
      return fail(PA_ERR_UNSUPPORTED, "no kernel for G=" + std::to_string(G));
    if (static_cast<int64_t>(num_seqs) * d.num_kv_heads > INT32_MAX)
      return fail(PA_ERR_UNSUPPORTED, "num_seqs * num_kv_heads must fit in 31 bits");
    if (max_query_len <= 0) return fail(PA_ERR_INVALID_ARG, "max_query_len must be positive");
    if (max_query_len > pa::prefill_max_query_len(G))
      return fail(PA_ERR_UNSUPPORTED, "max_query_len above " + std::to_string(pa::prefill_max_query_len(G)));
    if (!q || !out || !query_start || !block_tables || !context_lens)
      return fail(PA_ERR_INVALID_ARG, "NULL device pointer");
    if (!aligned16(q) || !aligned16(out)) return fail(PA_ERR_INVALID_ARG, "q and out must be 16-byte aligned");
    if (max_blocks_per_seq <= 0 || max_context_len <= 0)
      return fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq and max_context_len must be positive");
    if (!std::isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "scale must be finite");
    const int bs = d.block_size;
    const int64_t cap64 = std::min<int64_t>(max_context_len, static_cast<int64_t>(max_blocks_per_seq) * bs);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (debug_enabled()) {
      std::vector<int32_t> hc(num_seqs), hq(num_seqs + 1), ht(static_cast<size_t>(num_seqs) * max_blocks_per_seq);
      hipError_t e = hipMemcpyAsync(hc.data(), context_lens, sizeof(int32_t) * num_seqs, hipMemcpyDeviceToHost, s);
      if (e == hipSuccess)
        e = hipMemcpyAsync(hq.data(), query_start, sizeof(int32_t) * (num_seqs + 1), hipMemcpyDeviceToHost, s);
      if (e == hipSuccess)
        e = hipMemcpyAsync(ht.data(), block_tables, sizeof(int32_t) * ht.size(), hipMemcpyDeviceToHost, s);
      if (e == hipSuccess) e = hipStreamSynchronize(s);
      if (e != hipSuccess) return hip_fail(e, "PA_DEBUG readback");
      if (hq[0] != 0 || hq[num_seqs] > num_query_tokens)
        return fail(PA_ERR_INVALID_ARG, "query_start must start at 0 and end within num_query_tokens");
      for (int i = 0; i < num_seqs; ++i) {
        const int n = hq[i + 1] - hq[i];
        if (n < 0 || n > max_query_len || n > hc[i])
          return fail(PA_ERR_INVALID_ARG, "new tokens of sequence " + std::to_string(i) + " out of range");
        if (hc[i] < 1 || hc[i] > cap64)
          return fail(PA_ERR_INVALID_ARG, "context_lens[" + std::to_string(i) + "] out of range");
        const int nb = (hc[i] + bs - 1) / bs;
        for (int b = 0; b < nb; ++b) {
          const int32_t id = ht[static_cast<size_t>(i) * max_blocks_per_seq + b];
          if (id < 0 || id >= d.num_blocks)
            return fail(PA_ERR_INVALID_ARG, "block_tables[" + std::to_string(i) + "][" + std::to_string(b) + "] invalid");
        }
      }
    }
    pa::PrefillParams p{};
    p.pool = pool->buf;
    p.layer_off = static_cast<size_t>(layer) * d.num_blocks * d.num_kv_heads * 2 * static_cast<size_t>(bs) * d.head_dim;
    p.N = d.num_blocks;
    p.H = d.num_kv_heads;
    p.bs = bs;
    p.q = q;
    p.out = out;
    p.query_start = query_start;
    p.num_q_tokens = num_query_tokens;
    p.max_query_len = max_query_len;
    p.tables = block_tables;
    p.max_blocks = max_blocks_per_seq;
    p.ctx = context_lens;
    p.S = num_seqs;
    p.Hq = num_q_heads;
    p.G = G;
    p.ctx_cap = static_cast<int>(cap64);
    p.scale_log2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
    hipError_t e = pa::launch_prefill(p, d.dtype, d.head_dim, s);
    return e == hipSuccess ? PA_OK : hip_fail(e, "prefill launch");
  });
}

int pa_copy_blocks(pa_pool* pool, const int32_t* pairs, int n, void* stream) {
  return guarded([&]() -> int {
    if (!pool) return fail(PA_ERR_INVALID_ARG, "pool is NULL");
    if (n < 0) return fail(PA_ERR_INVALID_ARG, "pair count cannot be negative");
    if (n == 0) return PA_OK;
    if (!pairs) return fail(PA_ERR_INVALID_ARG, "pairs is NULL");
    if (n > 65535) return fail(PA_ERR_UNSUPPORTED, "at most 65535 pairs per call");
    hipError_t e = pa::launch_copy_blocks(geom_of(pool), pairs, n, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : hip_fail(e, "copy_blocks launch");
  });
}

size_t pa_host_block_bytes(const pa_pool* pool) {
  if (!pool) return 0;
  const pa_pool_desc& d = pool->desc;
  return static_cast<size_t>(d.num_layers) * d.num_kv_heads * 2 * static_cast<size_t>(d.block_size) * d.head_dim *
         elem_bytes(d.dtype);
}

int pa_host_tier_init(pa_pool* pool, int num_host_blocks) {
  return guarded([&]() -> int {
    if (!pool) return fail(PA_ERR_INVALID_ARG, "pool is NULL");
    std::string err;
    return alloc_status(pool->alloc.host_tier(num_host_blocks, &err), err);
  });
}

namespace {
int swap_seq(pa_pool* pool, int seq, int32_t* pairs_out, int cap_pairs, int* n_pairs, bool out) {
  if (!pool || !n_pairs) return fail(PA_ERR_INVALID_ARG, "NULL argument");
  *n_pairs = 0;
  auto& a = pool->alloc;
  if (!a.live(seq)) return fail(PA_ERR_INVALID_ARG, "unknown or released sequence");
  const size_t need = out ? (a.swapped(seq) ? 0 : a.table(seq).size()) : a.host_table(seq).size();
  if (static_cast<int64_t>(need) > cap_pairs) return fail(PA_ERR_BUFFER_TOO_SMALL, "pair capacity too small");
  if (need > 0 && !pairs_out) return fail(PA_ERR_INVALID_ARG, "pairs_out is NULL");
  std::vector<int32_t> pairs;
  std::string err;
  const pa::AllocResult r = out ? a.swap_out(seq, &pairs, &err) : a.swap_in(seq, &pairs, &err);
  if (r != pa::AllocResult::Ok) return alloc_status(r, err);
  std::copy(pairs.begin(), pairs.end(), pairs_out);
  *n_pairs = static_cast<int>(pairs.size() / 2);
  return PA_OK;
}
}  // namespace

int pa_seq_swap_out(pa_pool* pool, int seq, int32_t* pairs_out, int cap_pairs, int* n_pairs) {
  return guarded([&]() -> int { return swap_seq(pool, seq, pairs_out, cap_pairs, n_pairs, true); });
}

int pa_seq_swap_in(pa_pool* pool, int seq, int32_t* pairs_out, int cap_pairs, int* n_pairs) {
  return guarded([&]() -> int { return swap_seq(pool, seq, pairs_out, cap_pairs, n_pairs, false); });
}

int pa_swap_blocks(pa_pool* pool, const int32_t* pairs, int n, void* host_buf, size_t host_bytes, int direction,
                   void* stream) {
  return guarded([&]() -> int {
    if (!pool) return fail(PA_ERR_INVALID_ARG, "pool is NULL");
    if (n < 0) return fail(PA_ERR_INVALID_ARG, "pair count cannot be negative");
    if (direction != 0 && direction != 1) return fail(PA_ERR_INVALID_ARG, "direction must be 0 (out) or 1 (in)");
    if (n == 0) return PA_OK;
    if (!pairs || !host_buf) return fail(PA_ERR_INVALID_ARG, "NULL pointer");
    if (reinterpret_cast<uintptr_t>(host_buf) & 15u) return fail(PA_ERR_INVALID_ARG, "host buffer must be 16-byte aligned");
    // The kernel reads and writes the host buffer directly: it must be pinned
    // host memory the device can address.
    void* dev_view = nullptr;
    hipError_t e = hipHostGetDevicePointer(&dev_view, host_buf, 0);
    if (e != hipSuccess || !dev_view) {
      (void)hipGetLastError();
      return fail(PA_ERR_INVALID_ARG, "host buffer is not pinned host memory");
    }
    const size_t hbb = pa_host_block_bytes(pool);
    const int64_t host_blocks = static_cast<int64_t>(host_bytes / hbb);
    e = pa::launch_swap_blocks(geom_of(pool), pairs, n, dev_view, host_blocks, direction,
                               static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : hip_fail(e, "swap_blocks launch");
  });
}

int pa_probe_read_chunks(const void* buf, size_t buf_bytes, const int32_t* chunk_ids, int num_chunks,
                         int load_form, int wg_per_cu, int in_flight, void* sink, void* stream) {
  return guarded([&]() -> int {
    if (num_chunks < 0) return fail(PA_ERR_INVALID_ARG, "chunk count cannot be negative");
    if (!pa::probe_supported(load_form, wg_per_cu, in_flight))
      return fail(PA_ERR_UNSUPPORTED, "load_form 0-4, wg_per_cu 1-4, in_flight 1, 2 or 4 (1 or 2 into LDS)");
    if (num_chunks == 0) return PA_OK;
    if (!buf || !chunk_ids || !sink) return fail(PA_ERR_INVALID_ARG, "NULL device pointer");
    if (!aligned16(buf)) return fail(PA_ERR_INVALID_ARG, "buf must be 16-byte aligned");
    const int64_t nchunks_buf = static_cast<int64_t>(buf_bytes / 8192);
    if (nchunks_buf == 0) return fail(PA_ERR_INVALID_ARG, "buf holds no whole 8 KiB chunk");
    hipError_t e = pa::launch_probe_read(buf, nchunks_buf, chunk_ids, num_chunks, load_form, wg_per_cu, in_flight,
                                         sink, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : hip_fail(e, "probe launch");
  });
}

int pa_seq_create(pa_pool* pool, int* seq) {
  return guarded([&]() -> int {
    if (!pool || !seq) return fail(PA_ERR_INVALID_ARG, "NULL argument");
    *seq = pool->alloc.create();
    return PA_OK;
  });
}

int pa_seq_append(pa_pool* pool, int seq, int n_tokens, int32_t* slots_out, int32_t* cow_pairs_out,
                  int* n_cow) {
  return guarded([&]() -> int {
    if (!pool) return fail(PA_ERR_INVALID_ARG, "pool is NULL");
    if (n_tokens > 0 && !slots_out) return fail(PA_ERR_INVALID_ARG, "slots_out is NULL");
    std::string err;
    return alloc_status(pool->alloc.append(seq, n_tokens, slots_out, cow_pairs_out, n_cow, &err), err);
  });
}

int pa_seq_append_tokens(pa_pool* pool, int seq, const int32_t* token_ids, int n_tokens, int32_t* slots_out,
                         int32_t* cow_pairs_out, int* n_cow, int* n_cached) {
  return guarded([&]() -> int {
    if (!pool) return fail(PA_ERR_INVALID_ARG, "pool is NULL");
    if (n_tokens > 0 && (!slots_out || !token_ids)) return fail(PA_ERR_INVALID_ARG, "NULL argument");
    std::string err;
    return alloc_status(
        pool->alloc.append_tokens(seq, token_ids, n_tokens, slots_out, cow_pairs_out, n_cow, n_cached, &err), err);
  });
}

int pa_prefix_cache_enable(pa_pool* pool, int enable) {
  return guarded([&]() -> int {
    if (!pool) return fail(PA_ERR_INVALID_ARG, "pool is NULL");
    pool->alloc.enable_prefix_cache(enable != 0);
    return PA_OK;
  });
}

int pa_prefix_cache_stats(const pa_pool* pool, pa_prefix_stats* out) {
  return guarded([&]() -> int {
    if (!pool || !out) return fail(PA_ERR_INVALID_ARG, "NULL argument");
    const auto& c = pool->alloc.cache_counts();
    out->cached_blocks = pool->alloc.cached_blocks();
    out->registered = c.registered;
    out->hit_blocks = c.hit_blocks;
    out->evicted = c.evicted;
    out->lookups = c.lookups;
    return PA_OK;
  });
}

int pa_seq_fork(pa_pool* pool, int parent, int* child) {
  return guarded([&]() -> int {
    if (!pool || !child) return fail(PA_ERR_INVALID_ARG, "NULL argument");
    std::string err;
    return alloc_status(pool->alloc.fork(parent, child, &err), err);
  });
}

int pa_seq_release(pa_pool* pool, int seq) {
  return guarded([&]() -> int {
    if (!pool) return fail(PA_ERR_INVALID_ARG, "pool is NULL");
    std::string err;
    return alloc_status(pool->alloc.release(seq, &err), err);
  });
}

int pa_seq_block_table(const pa_pool* pool, int seq, int32_t* out, int cap, int* n, int* len_tokens) {
  return guarded([&]() -> int {
    if (!pool || !n) return fail(PA_ERR_INVALID_ARG, "NULL argument");
    if (!pool->alloc.live(seq)) return fail(PA_ERR_INVALID_ARG, "unknown or released sequence");
    const auto& t = pool->alloc.table(seq);
    *n = static_cast<int>(t.size());
    if (len_tokens) *len_tokens = pool->alloc.length(seq);
    if (static_cast<int>(t.size()) > cap) return fail(PA_ERR_BUFFER_TOO_SMALL, "table capacity too small");
    if (!t.empty() && !out) return fail(PA_ERR_INVALID_ARG, "out is NULL");
    std::copy(t.begin(), t.end(), out);
    return PA_OK;
  });
}

int pa_batch_tables(const pa_pool* pool, const int* seqs, int num_seqs, int max_blocks,
                    int32_t* tables_out, int32_t* context_lens_out) {
  return guarded([&]() -> int {
    if (!pool || (num_seqs > 0 && (!seqs || !tables_out || !context_lens_out)))
      return fail(PA_ERR_INVALID_ARG, "NULL argument");
    if (num_seqs < 0 || max_blocks < 0) return fail(PA_ERR_INVALID_ARG, "negative size");
    for (int i = 0; i < num_seqs; ++i) {
      if (!pool->alloc.live(seqs[i])) return fail(PA_ERR_INVALID_ARG, "unknown or released sequence");
      if (pool->alloc.swapped(seqs[i])) return fail(PA_ERR_INVALID_ARG, "sequence is swapped out");
      if (static_cast<int>(pool->alloc.table(seqs[i]).size()) > max_blocks)
        return fail(PA_ERR_BUFFER_TOO_SMALL, "max_blocks too small");
    }
    for (int i = 0; i < num_seqs; ++i) {
      const auto& t = pool->alloc.table(seqs[i]);
      int32_t* row = tables_out + static_cast<size_t>(i) * max_blocks;
      std::fill(row, row + max_blocks, -1);
      std::copy(t.begin(), t.end(), row);
      context_lens_out[i] = pool->alloc.length(seqs[i]);
    }
    return PA_OK;
  });
}

int pa_pool_state(const pa_pool* pool, int32_t* refcounts, int32_t* free_stack, int* n_free) {
  return guarded([&]() -> int {
    if (!pool || !n_free) return fail(PA_ERR_INVALID_ARG, "NULL argument");
    const auto& rc = pool->alloc.refcounts();
    const auto& st = pool->alloc.free_stack();
    if (refcounts) std::copy(rc.begin(), rc.end(), refcounts);
    if (free_stack) std::copy(st.begin(), st.end(), free_stack);
    *n_free = static_cast<int>(st.size());
    return PA_OK;
  });
}

int pa_pool_stats(const pa_pool* pool, pa_stats* s) {
  return guarded([&]() -> int {
    if (!pool || !s) return fail(PA_ERR_INVALID_ARG, "NULL argument");
    const auto& a = pool->alloc;
    s->num_blocks = a.num_blocks();
    s->free_blocks = static_cast<int64_t>(a.free_stack().size());
    s->used_blocks = s->num_blocks - s->free_blocks;
    s->shared_blocks = a.shared_blocks();
    s->cow_copies = a.cow_copies();
    s->live_seqs = a.live_seqs();
    s->logical_tokens = a.logical_tokens();
    s->tail_slots = a.tail_slots();
    return PA_OK;
  });
}

int pa_slots_for_positions(const int32_t* tables, int num_seqs, int max_blocks, int block_size,
                           const int32_t* pos_begin, const int32_t* n_tokens, int32_t* slots_out) {
  return guarded([&]() -> int {
    if (num_seqs < 0 || max_blocks < 0 || block_size <= 0) return fail(PA_ERR_INVALID_ARG, "bad size");
    if (num_seqs > 0 && (!tables || !pos_begin || !n_tokens || !slots_out))
      return fail(PA_ERR_INVALID_ARG, "NULL argument");
    size_t o = 0;
    for (int i = 0; i < num_seqs; ++i) {
      if (pos_begin[i] < 0 || n_tokens[i] < 0) return fail(PA_ERR_INVALID_ARG, "negative position or count");
      const int64_t end = static_cast<int64_t>(pos_begin[i]) + n_tokens[i];
      if (end > static_cast<int64_t>(max_blocks) * block_size)
        return fail(PA_ERR_INVALID_ARG, "position beyond the table of sequence " + std::to_string(i));
      const int32_t* row = tables + static_cast<size_t>(i) * max_blocks;
      for (int64_t pos = pos_begin[i]; pos < end; ++pos) {
        const int32_t b = row[pos / block_size];
        if (b < 0) return fail(PA_ERR_INVALID_ARG, "position maps to an empty table entry");
        slots_out[o++] = b * block_size + static_cast<int32_t>(pos % block_size);
      }
    }
    return PA_OK;
  });
}

}  // extern "C"
