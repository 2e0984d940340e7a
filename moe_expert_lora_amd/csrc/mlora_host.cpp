// Host-side integer work of libmlora.so: the route decision, the two per-row
// adapter maps, expert-table packing and the window split. Plain C++, no GPU.
//
// Sources: the "moe_row_adapter.rs" source page (route decision, refusal,
// adapter maps) and the "moe_lora_grouped" module index page (packing,
// windows, tile count, row token).
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <vector>

#include "mlora.h"
#include "mlora_internal.h"

namespace mlora {
namespace {
thread_local char g_err[512] = "";
constexpr int32_t kMaxExpertId = (1 << 24) - 1;
constexpr int32_t kMaxAdapterSlot = (1 << 16) - 1;
}  // namespace

int32_t fail(int32_t code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

void clear_error() { g_err[0] = '\0'; }

const char* last_error() { return g_err; }

}  // namespace mlora

using mlora::fail;

extern "C" {

const char* mlora_last_error(void) { return mlora::last_error(); }

int32_t mlora_m_tile(void) { return MLORA_MLG_M_TILE; }

int32_t mlora_resolve_moe_lora_route(int32_t adapter_slot, int32_t active,
                                     int32_t has_moe_lora) {
  if (!has_moe_lora) return MLORA_ROUTE_FOLD;
  if (adapter_slot < 0) return MLORA_ROUTE_SKIP;
  return adapter_slot == active ? MLORA_ROUTE_FOLD : MLORA_ROUTE_REFUSE;
}

int32_t mlora_ensure_decode_route_servable(int32_t route) {
  if (route == MLORA_ROUTE_FOLD || route == MLORA_ROUTE_SKIP) {
    mlora::clear_error();
    return MLORA_OK;
  }
  if (route == MLORA_ROUTE_REFUSE)
    return fail(MLORA_ERR_REFUSE,
                "MoE LoRA decode refused: a request names an adapter whose expert tables are "
                "not installed (only the active adapter's are); folding it would apply the "
                "wrong weights, so it must be served in a batch of its own");
  return fail(MLORA_ERR_INVALID, "ensure_decode_route_servable: %d is not a route", route);
}

int32_t mlora_pack_expert_tables(const int32_t* expert_ids, const uint64_t* a_addrs,
                                 const uint64_t* b_addrs, const float* scales,
                                 int64_t n_entries, uint64_t* a_table, uint64_t* b_table,
                                 float* scale_table, int64_t table_cap, int32_t* n_experts) {
  if (n_entries < 0) return fail(MLORA_ERR_INVALID, "pack_expert_tables: n_entries < 0");
  if (n_entries == 0) {
    mlora::clear_error();
    return MLORA_NONE;
  }
  if (!expert_ids || !a_addrs || !b_addrs || !scales || !n_experts)
    return fail(MLORA_ERR_INVALID, "pack_expert_tables: NULL input");
  int32_t max_id = -1;
  for (int64_t i = 0; i < n_entries; ++i) {
    const int32_t e = expert_ids[i];
    if (e < 0 || e > mlora::kMaxExpertId)
      return fail(MLORA_ERR_INVALID, "pack_expert_tables: entry %lld has expert id %d "
                  "outside [0, 2^24)", (long long)i, e);
    if (e > max_id) max_id = e;
  }
  const int64_t n = (int64_t)max_id + 1;
  if (table_cap < n) {
    *n_experts = (int32_t)n;
    return fail(MLORA_ERR_CAPACITY, "pack_expert_tables: %lld cells needed, capacity %lld",
                (long long)n, (long long)table_cap);
  }
  if (!a_table || !b_table || !scale_table)
    return fail(MLORA_ERR_INVALID, "pack_expert_tables: NULL table");
  for (int64_t e = 0; e < n; ++e) {
    a_table[e] = 0;
    b_table[e] = 0;
    scale_table[e] = 0.0f;
  }
  // Entries in input order: a later entry for the same id overwrites.
  for (int64_t i = 0; i < n_entries; ++i) {
    const int32_t e = expert_ids[i];
    a_table[e] = a_addrs[i];
    b_table[e] = b_addrs[i];
    scale_table[e] = scales[i];
  }
  *n_experts = (int32_t)n;
  mlora::clear_error();
  return MLORA_OK;
}

int32_t mlora_resolve_moe_lora_route_multi(int32_t adapter_slot, int32_t n_adapters) {
  if (adapter_slot < 0) return MLORA_ROUTE_SKIP;
  return adapter_slot < n_adapters ? MLORA_ROUTE_FOLD : MLORA_ROUTE_REFUSE;
}

int32_t mlora_build_moe_row_adapter_decode_multi(const int32_t* adapter_slots, int64_t n_slots,
                                                 int64_t padded_n, int32_t n_adapters,
                                                 int32_t* out) {
  if (n_slots < 0 || padded_n < 0 || n_adapters < 0)
    return fail(MLORA_ERR_INVALID, "build_moe_row_adapter_decode_multi: negative size");
  if ((n_slots > 0 && padded_n > 0 && !adapter_slots) || (padded_n > 0 && !out))
    return fail(MLORA_ERR_INVALID, "build_moe_row_adapter_decode_multi: NULL pointer");
  for (int64_t i = 0; i < padded_n; ++i) {
    const int32_t s = i < n_slots ? adapter_slots[i] : -1;
    out[i] = mlora_resolve_moe_lora_route_multi(s, n_adapters) == MLORA_ROUTE_FOLD ? s : -1;
  }
  mlora::clear_error();
  return MLORA_OK;
}

int32_t mlora_pack_expert_tables_multi(const int32_t* adapter_slots, const int32_t* expert_ids,
                                       const uint64_t* a_addrs, const uint64_t* b_addrs,
                                       const float* scales, int64_t n_entries,
                                       uint64_t* a_table, uint64_t* b_table, float* scale_table,
                                       int64_t table_cap, int32_t* n_adapters,
                                       int32_t* n_experts) {
  const char* who = "pack_expert_tables_multi";
  if (n_entries < 0) return fail(MLORA_ERR_INVALID, "%s: n_entries < 0", who);
  if (n_entries == 0) {
    mlora::clear_error();
    return MLORA_NONE;
  }
  if (!adapter_slots || !expert_ids || !a_addrs || !b_addrs || !scales || !n_adapters ||
      !n_experts)
    return fail(MLORA_ERR_INVALID, "%s: NULL input", who);
  int32_t max_slot = -1, max_id = -1;
  for (int64_t i = 0; i < n_entries; ++i) {
    const int32_t sl = adapter_slots[i], e = expert_ids[i];
    if (sl < 0 || sl > mlora::kMaxAdapterSlot || e < 0 || e > mlora::kMaxExpertId)
      return fail(MLORA_ERR_INVALID, "%s: entry %lld has slot %d / expert id %d outside "
                  "[0, 2^16) / [0, 2^24)", who, (long long)i, sl, e);
    if (sl > max_slot) max_slot = sl;
    if (e > max_id) max_id = e;
  }
  const int64_t na = (int64_t)max_slot + 1, ne = (int64_t)max_id + 1, cells = na * ne;
  if (cells > 0x7fffffffll)
    return fail(MLORA_ERR_INVALID, "%s: %lld x %lld cells", who, (long long)na, (long long)ne);
  if (table_cap < cells) {
    *n_adapters = (int32_t)na;
    *n_experts = (int32_t)ne;
    return fail(MLORA_ERR_CAPACITY, "%s: %lld cells needed, capacity %lld", who,
                (long long)cells, (long long)table_cap);
  }
  if (!a_table || !b_table || !scale_table) return fail(MLORA_ERR_INVALID, "%s: NULL table", who);
  for (int64_t c = 0; c < cells; ++c) {
    a_table[c] = 0;
    b_table[c] = 0;
    scale_table[c] = 0.0f;
  }
  // Entries in input order: a later entry for the same (slot, id) overwrites.
  for (int64_t i = 0; i < n_entries; ++i) {
    const int64_t c = (int64_t)adapter_slots[i] * ne + expert_ids[i];
    a_table[c] = a_addrs[i];
    b_table[c] = b_addrs[i];
    scale_table[c] = scales[i];
  }
  *n_adapters = (int32_t)na;
  *n_experts = (int32_t)ne;
  mlora::clear_error();
  return MLORA_OK;
}

int32_t mlora_build_moe_row_adapter_host(const int32_t* cu_seqlens, int64_t n_cu,
                                         const int32_t* adapter_slots, int64_t n_slots,
                                         int32_t* out, int64_t out_cap, int64_t* total) {
  if (n_cu < 0 || n_slots < 0 || !total)
    return fail(MLORA_ERR_INVALID, "build_moe_row_adapter_host: bad sizes or NULL total");
  if (n_cu < 2) return fail(MLORA_NONE, "build_moe_row_adapter_host: fewer than 2 boundaries");
  if (!cu_seqlens) return fail(MLORA_ERR_INVALID, "build_moe_row_adapter_host: NULL cu_seqlens");
  const int64_t batch = n_cu - 1;
  if (n_slots != batch)
    return fail(MLORA_NONE, "build_moe_row_adapter_host: %lld slots for %lld streams",
                (long long)n_slots, (long long)batch);
  if (cu_seqlens[0] != 0)
    return fail(MLORA_NONE, "build_moe_row_adapter_host: first boundary is not 0");
  // The boundaries must be a non-decreasing prefix sum; the map's length is
  // the last one, so none is trusted before all are checked.
  for (int64_t b = 0; b < batch; ++b) {
    if (cu_seqlens[b + 1] < cu_seqlens[b])
      return fail(MLORA_NONE, "build_moe_row_adapter_host: boundary %lld decreases",
                  (long long)(b + 1));
  }
  const int64_t n = cu_seqlens[batch];
  if (out_cap < n) {
    *total = n;
    return fail(MLORA_ERR_CAPACITY, "build_moe_row_adapter_host: %lld entries needed, "
                "capacity %lld", (long long)n, (long long)out_cap);
  }
  if (n > 0 && (!out || !adapter_slots))
    return fail(MLORA_ERR_INVALID, "build_moe_row_adapter_host: NULL out or slots");
  for (int64_t b = 0; b < batch; ++b)
    for (int32_t t = cu_seqlens[b]; t < cu_seqlens[b + 1]; ++t) out[t] = adapter_slots[b];
  *total = n;
  mlora::clear_error();
  return MLORA_OK;
}

int32_t mlora_build_moe_row_adapter_decode(const int32_t* adapter_slots, int64_t n_slots,
                                           int64_t padded_n, int32_t active,
                                           int32_t has_moe_lora, int32_t* out) {
  if (n_slots < 0 || padded_n < 0)
    return fail(MLORA_ERR_INVALID, "build_moe_row_adapter_decode: negative size");
  if (padded_n > 0 && !out)
    return fail(MLORA_ERR_INVALID, "build_moe_row_adapter_decode: NULL out");
  const int64_t live = n_slots < padded_n ? n_slots : padded_n;
  if (live > 0 && !adapter_slots)
    return fail(MLORA_ERR_INVALID, "build_moe_row_adapter_decode: NULL slots");
  for (int64_t i = 0; i < padded_n; ++i) {
    int32_t v = -1;
    if (i < live &&
        mlora_resolve_moe_lora_route(adapter_slots[i], active, has_moe_lora) == MLORA_ROUTE_FOLD)
      v = active;
    out[i] = v;
  }
  mlora::clear_error();
  return MLORA_OK;
}

int32_t mlora_grouped_down_windows(int64_t total_rows, int64_t cap, int64_t* starts,
                                   int64_t* ends, int64_t out_cap, int64_t* n_windows) {
  if (cap <= 0) return fail(MLORA_ERR_INVALID, "grouped_down_windows: cap must be positive");
  if (total_rows < 0 || !n_windows)
    return fail(MLORA_ERR_INVALID, "grouped_down_windows: negative rows or NULL count");
  const int64_t count = total_rows / cap + (total_rows % cap != 0);
  if (out_cap < count) {
    *n_windows = count;
    return fail(MLORA_ERR_CAPACITY, "grouped_down_windows: %lld windows, capacity %lld",
                (long long)count, (long long)out_cap);
  }
  if (count > 0 && (!starts || !ends))
    return fail(MLORA_ERR_INVALID, "grouped_down_windows: NULL output");
  for (int64_t w = 0; w < count; ++w) {
    starts[w] = w * cap;
    ends[w] = (w + 1) * cap < total_rows ? (w + 1) * cap : total_rows;
  }
  *n_windows = count;
  mlora::clear_error();
  return MLORA_OK;
}

uint32_t mlora_grouped_down_wc(int64_t row_offset, int64_t row_end) {
  const int64_t len = row_end - row_offset;
  if (len <= 0) return 1;
  const int64_t tiles = (len + MLORA_MLG_M_TILE - 1) / MLORA_MLG_M_TILE;
  return tiles > 0xFFFFFFFFll ? 0xFFFFFFFFu : (uint32_t)tiles;
}

int32_t mlora_gather_row_token(int32_t row, int32_t top_k) {
  if (row < 0 || top_k <= 0) return -1;
  return row / top_k;
}

}  // extern "C"
