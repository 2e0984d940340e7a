/*
 * mlora.h - C ABI of libmlora.so: the MoE expert-LoRA fold on AMD Instinct
 * MI355X (gfx950), and the host-side integer work around it.
 *
 * The fold adds, in place, each routed expert's low-rank delta onto the base
 * projection output of a (token, slot) row:
 *
 *     base_out[row] += scale_e * ((x[token(row)] @ A_e^T) @ B_e^T)
 *
 * (the two fold items of the "moe_lora_grouped" launcher-module index page).
 * Sources cited below:
 *   [P1] the "moe_row_adapter.rs" source page (GPU-free MoE LoRA routing),
 *   [P2] the "moe_lora_grouped" module index page (fold launchers, packing).
 *
 * Conventions shared by every entry point:
 *   - Every buffer, host or device, belongs to the caller. The library never
 *     allocates, frees or synchronises, and keeps no state except a
 *     thread-local last-error message (mlora_last_error) and the launch-shape
 *     overrides below.
 *   - Host outputs are written only when the call returns MLORA_OK (or, for
 *     sizes, MLORA_ERR_CAPACITY, which writes only the needed size).
 *   - The two fold calls enqueue kernels on the caller's stream and return at
 *     once. The host never reads routing data, so a fold is capturable in a
 *     HIP graph. A device-side fault surfaces at the caller's next sync.
 *   - Layouts are row-major and contiguous. bf16 is stored as its 16 raw bits.
 *   - Environment variables named MLORA_* override launch shapes (rows and
 *     columns per workgroup, launches per call). They exist for measurement:
 *     no value changes what a call computes beyond the rounding differences
 *     documented for the two-kernel gather, and no value changes the size a
 *     workspace query returns. They are read once per process, at the first
 *     fold call, and again only by mlora_reload_launch_overrides; no fold
 *     call reads the environment.
 */
#ifndef MLORA_H_
#define MLORA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
enum {
  MLORA_OK = 0,
  MLORA_NONE = 1,           /* the pages' "None": nothing was written         */
  MLORA_ERR_INVALID = -1,   /* bad arguments (also the pages' panic on cap 0) */
  MLORA_ERR_REFUSE = -2,    /* a decode batch the single-active fold refuses  */
  MLORA_ERR_CAPACITY = -3,  /* a host output is too small; size written       */
  MLORA_ERR_HIP = -4        /* the HIP runtime rejected a launch              */
};

/* Per-request fold decision [P1 resolve_moe_lora_route; MoeLoraRoute]. */
enum { MLORA_ROUTE_FOLD = 0, MLORA_ROUTE_SKIP = 1, MLORA_ROUTE_REFUSE = 2 };

/* Element type of x, A_e, B_e and base_out. */
enum { MLORA_F32 = 0, MLORA_BF16 = 1 };

/* Rows per grouped-fold tile [P2 MLG_M_TILE]: the host grid
 * (mlora_grouped_down_wc) and the kernel's tiles use this one value. */
#define MLORA_MLG_M_TILE 64

/*
 * Device tables of one projection's expert LoRA pairs, indexed by expert id
 * [P2 MoeExpertRoute]. a_table[e] / b_table[e] hold the device addresses of
 * A_e [max_rank, k_in] and B_e [n_out, max_rank]; scale_table[e] is scale_e.
 * A cell of 0 marks an unadapted expert. All experts share k_in, n_out and
 * max_rank (a lower rank is zero-padded to max_rank). Every A_e / B_e address
 * must be 16-byte aligned. The struct itself lives in host memory; the three
 * table pointers are device pointers with n_experts entries.
 */
typedef struct mlora_expert_route {
  const uint64_t* a_table;
  const uint64_t* b_table;
  const float* scale_table;
  int32_t n_experts;
  int32_t k_in;      /* multiple of 8, >= 8                        */
  int32_t n_out;     /* multiple of 8, >= 8                        */
  int32_t max_rank;  /* 1 .. 128                                   */
  int32_t dtype;     /* MLORA_BF16 or MLORA_F32                    */
} mlora_expert_route;

/* ------------------------------------------------------------------------ */
/* Host-side integer work (no GPU needed).                                   */
/* ------------------------------------------------------------------------ */

/* [P1 resolve_moe_lora_route] With has_moe_lora == 0 every request folds;
 * otherwise a negative slot is Skip, slot == active is Fold, any other slot
 * is Refuse. Returns an MLORA_ROUTE_* value. */
int32_t mlora_resolve_moe_lora_route(int32_t adapter_slot, int32_t active,
                                     int32_t has_moe_lora);

/* [P1 ensure_decode_route_servable] MLORA_OK for Fold and Skip,
 * MLORA_ERR_REFUSE (message names the one-adapter-per-batch rule) for Refuse,
 * MLORA_ERR_INVALID for a value that is no route. */
int32_t mlora_ensure_decode_route_servable(int32_t route);

/* [P2 pack_expert_tables, ExpertTables] Pack n_entries entries
 * (expert_ids[i], a_addrs[i], b_addrs[i], scales[i]) into host tables indexed
 * by expert id, with n = max id + 1 cells, 0 / 0.0 at ids no entry names, and
 * the last entry winning for a repeated id. Ids must lie in [0, 2^24).
 *   n_entries == 0            -> MLORA_NONE, nothing written.
 *   a negative / too large id -> MLORA_ERR_INVALID, nothing written.
 *   table_cap < n             -> MLORA_ERR_CAPACITY, only *n_experts written.
 * The three tables may be NULL together with table_cap == 0 to query n.
 * Upload the tables to device memory to build an mlora_expert_route. */
int32_t mlora_pack_expert_tables(const int32_t* expert_ids, const uint64_t* a_addrs,
                                 const uint64_t* b_addrs, const float* scales,
                                 int64_t n_entries, uint64_t* a_table, uint64_t* b_table,
                                 float* scale_table, int64_t table_cap, int32_t* n_experts);

/* [P1 build_moe_row_adapter_host] Per-token adapter map of a packed prefill
 * batch: stream b's slot is copied unchanged onto tokens
 * cu_seqlens[b] .. cu_seqlens[b+1] (n_cu = batch + 1).
 *   MLORA_NONE (nothing written) when n_cu < 2, n_slots != n_cu - 1,
 *   cu_seqlens[0] != 0, or a boundary is negative or below its predecessor.
 *   MLORA_ERR_CAPACITY when out_cap < total (only *total written).
 * On MLORA_OK, out[0 .. total) holds the map and *total its length. The copy
 * is literal: a slot >= 0 that is not the active one would fold the active
 * adapter, so callers resolve routes first. */
int32_t mlora_build_moe_row_adapter_host(const int32_t* cu_seqlens, int64_t n_cu,
                                         const int32_t* adapter_slots, int64_t n_slots,
                                         int32_t* out, int64_t out_cap, int64_t* total);

/* [P1 build_moe_row_adapter_decode] Per-sequence adapter map of a decode batch:
 * out[i] (i < padded_n) is `active` when sequence i exists (i < n_slots) and
 * resolves to Fold, else -1 (Skip, Refuse and padding). Slots past padded_n
 * are ignored. out must hold padded_n entries. MLORA_ERR_INVALID for a
 * negative size or a NULL pointer that is needed. */
int32_t mlora_build_moe_row_adapter_decode(const int32_t* adapter_slots, int64_t n_slots,
                                           int64_t padded_n, int32_t active,
                                           int32_t has_moe_lora, int32_t* out);

/* [P2 grouped_down_windows] Contiguous [start, end) windows of at most cap
 * rows covering 0 .. total_rows, all full except the last; zero rows give no
 * window. cap <= 0 or total_rows < 0 -> MLORA_ERR_INVALID.
 * out_cap < count -> MLORA_ERR_CAPACITY (only *n_windows written). */
int32_t mlora_grouped_down_windows(int64_t total_rows, int64_t cap, int64_t* starts,
                                   int64_t* ends, int64_t out_cap, int64_t* n_windows);

/* [P2 grouped_down_wc] Row tiles of the window [row_offset, row_end):
 * ceil((row_end - row_offset) / MLORA_MLG_M_TILE), at least 1. */
uint32_t mlora_grouped_down_wc(int64_t row_offset, int64_t row_end);

/* [P2 gather_row_token] The token that owns flat (token, slot) row `row`:
 * row / top_k. Returns -1 when row < 0 or top_k <= 0. */
int32_t mlora_gather_row_token(int32_t row, int32_t top_k);

/* The grouped-fold tile rows (MLORA_MLG_M_TILE), for callers that cannot see
 * the macro. */
int32_t mlora_m_tile(void);

/* Message of the last failing call on this thread ("" if none). The string
 * stays valid until the next call on the same thread. */
const char* mlora_last_error(void);

/* ------------------------------------------------------------------------ */
/* Device folds (enqueue on `stream`, a hipStream_t; NULL = default stream).  */
/* ------------------------------------------------------------------------ */

/*
 * [P2 moe_lora_gather_bgmv] Decode fold over flat (token, slot) rows.
 * For every row in [0, n_slots): token = row / top_k; the row is skipped when
 * row_adapter[token] < 0 [P1 build_moe_row_adapter_decode], when
 * e = indices[row] is negative or >= n_experts, or when a_table[e] or
 * b_table[e] is 0 [P2 module invariant]. Otherwise
 *     base_out[row, :] = round(base_out[row, :] + scale_e * B_e (A_e x[token]))
 * with fp32 accumulation and, for bf16, one round-to-nearest-even store.
 * Skipped rows are not written at all.
 *
 * Device arguments:
 *   x           [n_tokens, k_in]   dtype (bf16 or f32), read only
 *   base_out    [n_slots, n_out]   dtype, updated in place
 *   indices     [n_slots]          int32 expert id per row, read on device
 *   row_adapter [n_tokens]         int32 per-token map, read on device
 * n_tokens must be >= ceil(n_slots / top_k). x and base_out must be 16-byte
 * aligned. n_slots == 0 or n_experts == 0 enqueues nothing.
 *
 * Workspace (device, caller-owned, optional): with workspace == NULL and
 * workspace_bytes == 0 the fold runs as one kernel. With a workspace of at
 * least mlora_gather_bgmv_workspace_bytes(n_slots, k_in, max_rank) bytes,
 * 256-byte aligned, calls whose k_in spans more than 16 k steps of 32 and
 * whose experts hold at most 64 rows on average run as two kernels (a shrink
 * split over k ranges into the workspace, then the expand), which spreads each
 * expert's A_e over more workgroups; other calls stay on one kernel. The two forms may differ in the
 * last bits (the k sums are grouped differently); both meet the same bound.
 * The contents need no initialisation and are dead once the call's kernels
 * finish; calls that share one workspace must be ordered (one stream). An f32
 * route ignores it.
 * Returns MLORA_OK, MLORA_ERR_INVALID (arguments; nothing enqueued, including
 * a misaligned or NULL-with-size workspace), MLORA_ERR_CAPACITY (workspace too
 * small; nothing enqueued) or MLORA_ERR_HIP (launch rejected).
 */
int32_t mlora_gather_bgmv(const mlora_expert_route* route, const void* x, int64_t n_tokens,
                          void* base_out, const int32_t* indices, const int32_t* row_adapter,
                          int64_t n_slots, int32_t top_k, void* workspace,
                          uint64_t workspace_bytes, void* stream);

/*
 * [P2 MoeExpertRoute, moe_lora_gather_bgmv] One gather call of a set: a
 * projection's route and its operands. A MoE layer builds one route per
 * projection (gate, up, down) and the router fold a one-entry route; a set
 * folds several such projections in one launch.
 *   x          device, x_rows rows of x_ld elements (x_ld >= k_in, a multiple
 *              of 8). With x_by_row == 0, flat row r reads x[r / top_k]
 *              (token-major, as mlora_gather_bgmv); with x_by_row == 1 it
 *              reads x[r] (slot-major: one row per (token, slot) row, the
 *              down projection's input), and x_rows must be >= n_slots.
 *   base_out   device, n_slots rows of out_ld elements (out_ld >= n_out, a
 *              multiple of 8): e.g. the gate and up halves of one
 *              [n_slots, 2 * n_out] tensor, each with out_ld = 2 * n_out.
 *   indices    device [n_slots] expert ids; row_adapter device [map_len]
 *              per-token map (map_len >= ceil(n_slots / top_k)); the skip
 *              rules of mlora_gather_bgmv apply, the map indexed by
 *              r / top_k in both x modes.
 * x and base_out must be 16-byte aligned.
 */
typedef struct mlora_projection {
  const mlora_expert_route* route;  /* host pointer                        */
  const void* x;
  int64_t x_rows;
  int64_t x_ld;
  int32_t x_by_row;
  void* base_out;
  int64_t out_ld;
  const int32_t* indices;
  const int32_t* row_adapter;
  int64_t map_len;
  int64_t n_slots;
  int32_t top_k;
} mlora_projection;

/*
 * [P2 MoeExpertRoute, moe_lora_gather_bgmv] The gather fold of 1 to 4
 * projections in one launch (the per-layer projection set): every
 * projection's rows are folded exactly as a mlora_gather_bgmv call without a
 * workspace would fold them, bit for bit, whatever the other projections in
 * the set. All projections must be bf16 and use the same number of rank
 * blocks (ceil(max_rank / 16) rounded up to 1, 2, 4 or 8); k_in, n_out,
 * routing and row counts may differ. Projections with no rows or no experts
 * contribute nothing. Their base_out regions must not overlap (one launch
 * writes them all). Returns MLORA_OK, MLORA_ERR_INVALID (nothing enqueued)
 * or MLORA_ERR_HIP.
 */
int32_t mlora_gather_bgmv_set(const mlora_projection* projs, int32_t n_proj, void* stream);

/* ------------------------------------------------------------------------ */
/* Several adapters at once (past the pages' single-active phase).           */
/* ------------------------------------------------------------------------ */
/*
 * A reading of [P1 resolve_moe_lora_route, ensure_decode_route_servable],
 * whose phase-1 design installs one adapter and refuses a decode batch that
 * asks for another, extended to several installed adapters: every adapter
 * slot s in [0, n_adapters) has its own expert tables [P2 ExpertTables], and
 * a row folds with the tables of its own token's slot.
 */

/* Route of one request: MLORA_ROUTE_SKIP for a negative slot, MLORA_ROUTE_FOLD
 * for a slot below n_adapters (its tables are installed), MLORA_ROUTE_REFUSE
 * otherwise (pass it to mlora_ensure_decode_route_servable to refuse). */
int32_t mlora_resolve_moe_lora_route_multi(int32_t adapter_slot, int32_t n_adapters);

/* Decode map: out[i] (i < padded_n) is sequence i's own slot when its route
 * is Fold, else -1 (Skip, Refuse, padding). MLORA_ERR_INVALID for a negative
 * size or a NULL pointer that is needed. */
int32_t mlora_build_moe_row_adapter_decode_multi(const int32_t* adapter_slots, int64_t n_slots,
                                                 int64_t padded_n, int32_t n_adapters,
                                                 int32_t* out);

/* [P2 pack_expert_tables] per slot: entries (adapter_slots[i], expert_ids[i],
 * a_addrs[i], b_addrs[i], scales[i]) into host tables of n_adapters x
 * n_experts cells, cell (s, e) at s * n_experts + e; n_adapters = max slot +
 * 1, n_experts = max id + 1; unnamed cells 0 / 0.0; the last entry wins for a
 * repeated (slot, id). Slots must lie in [0, 2^16), ids in [0, 2^24).
 * MLORA_NONE for no entries; MLORA_ERR_CAPACITY (only the two counts
 * written) when table_cap < n_adapters * n_experts (tables may then be
 * NULL); MLORA_ERR_INVALID for a bad slot or id. */
int32_t mlora_pack_expert_tables_multi(const int32_t* adapter_slots, const int32_t* expert_ids,
                                       const uint64_t* a_addrs, const uint64_t* b_addrs,
                                       const float* scales, int64_t n_entries,
                                       uint64_t* a_table, uint64_t* b_table, float* scale_table,
                                       int64_t table_cap, int32_t* n_adapters,
                                       int32_t* n_experts);

/* Device tables of several adapters' expert pairs: n_adapters * n_experts
 * cells, cell (s, e) at s * n_experts + e (as packed above); other fields as
 * in mlora_expert_route. */
typedef struct mlora_multi_route {
  const uint64_t* a_table;
  const uint64_t* b_table;
  const float* scale_table;
  int32_t n_adapters;
  int32_t n_experts;
  int32_t k_in;
  int32_t n_out;
  int32_t max_rank;
  int32_t dtype;     /* MLORA_BF16 only */
} mlora_multi_route;

/*
 * [P2 moe_lora_gather_bgmv] with several adapters: flat row r (token
 * t = r / top_k) folds with cell (row_adapter[t], indices[r]), and is skipped
 * when row_adapter[t] < 0 or >= n_adapters, when indices[r] is negative or
 * >= n_experts, or when the cell's a or b address is 0. Arithmetic, layouts
 * and the other rules as mlora_gather_bgmv without a workspace (one kernel;
 * with n_adapters == 1 and a map of 0 / -1, the same bits as
 * mlora_gather_bgmv on that slot's tables). Returns MLORA_OK,
 * MLORA_ERR_INVALID (nothing enqueued) or MLORA_ERR_HIP.
 */
int32_t mlora_gather_bgmv_multi(const mlora_multi_route* route, const void* x, int64_t n_tokens,
                                void* base_out, const int32_t* indices,
                                const int32_t* row_adapter, int64_t n_slots, int32_t top_k,
                                void* stream);

/* Bytes of workspace mlora_gather_bgmv may use: KC * n_slots * 64 * NB, KC =
 * clamp(ceil(ceil(k_in / 32) / 16), 1, 4) k ranges, NB = ceil(max_rank / 16)
 * rounded up to 1, 2, 4 or 8, rounded up to 256. 0 for n_slots <= 0 or invalid
 * k_in / max_rank. */
uint64_t mlora_gather_bgmv_workspace_bytes(int64_t n_slots, int32_t k_in, int32_t max_rank);

/*
 * [P2 moe_lora_grouped_down] Prefill fold over expert-sorted rows in the
 * window [row_offset, row_end) of a [n_rows, n_out] base_out.
 * The expert of sorted row r is the e with expert_offsets[e] <= r <
 * expert_offsets[e+1] (e < n_route; rows in no span are skipped). The row's
 * token is sorted_ids[r] / top_k, sorted_ids holding each sorted row's flat
 * (token, slot) id. Skip rules and arithmetic are those of mlora_gather_bgmv,
 * with row_adapter indexed by that token; a token outside [0, n_tokens) is
 * skipped. Rows outside the window are not touched. The device reads the
 * routing; expert_offsets must be non-decreasing (other contents stay in
 * bounds but fold unspecified rows of the window).
 *
 * Device arguments:
 *   x              [n_tokens, k_in]  dtype
 *   base_out       [n_rows, n_out]   dtype, updated in place
 *   expert_offsets [n_route + 1]     int32
 *   sorted_ids     [n_rows]          int32
 *   row_adapter    [n_tokens]        int32
 * 0 <= row_offset <= row_end <= n_rows. An empty window enqueues nothing.
 *
 * Workspace (device, caller-owned, optional): with workspace == NULL and
 * workspace_bytes == 0 the fold runs as one kernel. With a workspace of at
 * least mlora_grouped_down_workspace_bytes(row_offset, row_end, max_rank)
 * bytes, 256-byte aligned, it runs as two kernels (shrink into the workspace,
 * then expand), which streams base_out faster on large windows; both forms
 * give the same bits. The contents need no initialisation and are dead once
 * the call's kernels finish; calls that share one workspace must be ordered
 * (one stream). bf16 only uses it; an f32 route ignores it.
 * Returns MLORA_OK, MLORA_ERR_INVALID (arguments, including a misaligned or
 * NULL-with-size workspace), MLORA_ERR_CAPACITY (workspace too small;
 * nothing enqueued) or MLORA_ERR_HIP.
 */
int32_t mlora_grouped_down(const mlora_expert_route* route, const void* x, int64_t n_tokens,
                           void* base_out, int64_t n_rows, const int32_t* expert_offsets,
                           int32_t n_route, const int32_t* sorted_ids,
                           const int32_t* row_adapter, int32_t top_k, int64_t row_offset,
                           int64_t row_end, void* workspace, uint64_t workspace_bytes,
                           void* stream);

/*
 * Grouped fold of every sorted row, window by window: the windows are those of
 * mlora_grouped_down_windows(n_rows, cap), and the result equals calling
 * mlora_grouped_down on each of them in order with a workspace, bit for bit
 * (rows are independent). Consecutive windows are launched together, in
 * launches of whole windows holding at least 16384 rows (the override
 * MLORA_ALL_MIN_ROWS may lower the minimum to between 1 and 16384 rows; 1
 * launches one window at a time), and the launches are pipelined: one kernel expands launch l's rows
 * while it shrinks launch l + 1's, so a shrink overlaps the previous rows'
 * base_out traffic. Arguments as for mlora_grouped_down; cap <= 0 ->
 * MLORA_ERR_INVALID [P2 grouped_down_windows]. The workspace is required for
 * bf16 (two launch slots, see the size query below; NULL or too small ->
 * MLORA_ERR_CAPACITY, nothing enqueued); an f32 route folds the windows one
 * by one without it.
 */
int32_t mlora_grouped_down_all(const mlora_expert_route* route, const void* x, int64_t n_tokens,
                               void* base_out, int64_t n_rows, const int32_t* expert_offsets,
                               int32_t n_route, const int32_t* sorted_ids,
                               const int32_t* row_adapter, int32_t top_k, int64_t cap,
                               void* workspace, uint64_t workspace_bytes, void* stream);

/* Bytes of workspace mlora_grouped_down_all needs, whatever launch minimum
 * it runs with (the default, any override, or the one-window fallback taken
 * when a group of windows of base_out would pass 4 GiB): the largest, over
 * launches of m whole windows (m from 1 to ceil(16384 / cap)), of one slot
 * when L = min(n_rows, m * cap) rows cover every row and two slots
 * otherwise, a slot being mlora_grouped_down_workspace_bytes of L rows
 * rounded up to 256. Reads no environment. 0 for n_rows <= 0, cap <= 0 or
 * max_rank outside [1, 128]. */
uint64_t mlora_grouped_down_all_workspace_bytes(int64_t n_rows, int64_t cap, int32_t max_rank);

/*
 * [P2 module doc: the host-loop fold the device-routed launchers replace]
 * The sorted fold driven from the host: with the expert spans copied to the
 * host beforehand (expert_offsets_host, the caller's device-to-host copy of
 * expert_offsets) and the host copies of the packed tables, one
 * mlora_grouped_down launch per expert that has rows and both table cells,
 * over exactly its span. The result equals mlora_grouped_down over every row,
 * bit for bit (rows are independent). It exists as the baseline that shows
 * what reading the routing on the device buys: it needs the host copy (a
 * synchronisation of the caller's stream) and up to n_route launches, and
 * cannot be captured once for every routing. The workspace, if given, must
 * hold mlora_grouped_down_workspace_bytes of the largest span (the per-call
 * form's workspace rules apply). Spans outside [0, n_rows] or decreasing ->
 * MLORA_ERR_INVALID before any launch; other errors as mlora_grouped_down
 * (launches made before a failing one stay enqueued).
 */
int32_t mlora_apply_expert_lora_sorted(const mlora_expert_route* route, const void* x,
                                       int64_t n_tokens, void* base_out, int64_t n_rows,
                                       const int32_t* expert_offsets,
                                       const int32_t* expert_offsets_host, int32_t n_route,
                                       const uint64_t* a_table_host,
                                       const uint64_t* b_table_host, const int32_t* sorted_ids,
                                       const int32_t* row_adapter, int32_t top_k,
                                       void* workspace, uint64_t workspace_bytes, void* stream);

/* Bytes of workspace mlora_grouped_down needs for its two-kernel form on the
 * window [row_offset, row_end) at this max_rank: (row_end - row_offset) rows
 * of 64 * NB bytes, NB = ceil(max_rank / 16) rounded up to 1, 2, 4 or 8,
 * rounded up to 256, plus 8 bytes per row, rounded up to 256. 0 for an empty
 * window or invalid arguments (negative offsets, row_end < row_offset,
 * max_rank outside [1, 128]). */
uint64_t mlora_grouped_down_workspace_bytes(int64_t row_offset, int64_t row_end,
                                            int32_t max_rank);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the fold of
 * mlora_grouped_down_all, with the same arguments and the same bits, but no
 * workspace. Its two launch slots live in a static device array of
 * MLORA_NOALLOC_SCRATCH_BYTES bytes inside the library, one per device, held
 * until the process ends; its address is looked up once per device, at the
 * first call with that device current. The call allocates nothing.
 *   - A call needing more than MLORA_NOALLOC_SCRATCH_BYTES (the
 *     mlora_grouped_down_all_workspace_bytes figure of its launches; 32 MiB
 *     holds two slots of 16384 rows at max_rank 128) returns
 *     MLORA_ERR_CAPACITY, enqueues nothing and reads no device memory.
 *   - The stream (NULL = the default stream) must belong to the current
 *     device: otherwise MLORA_ERR_INVALID.
 *   - Every call on one device shares that device's array, and the array
 *     keeps the last call's contents; the fold needs no initialised contents
 *     (each launch writes every scratch entry it reads). Calls that overlap
 *     on one device, on different streams or from different threads without
 *     ordering, race on it and give undefined results.
 * Other errors are those of mlora_grouped_down_all. An f32 route uses no
 * scratch.
 */
#define MLORA_NOALLOC_SCRATCH_BYTES (32ull << 20)
int32_t mlora_grouped_down_all_noalloc(const mlora_expert_route* route, const void* x,
                                       int64_t n_tokens, void* base_out, int64_t n_rows,
                                       const int32_t* expert_offsets, int32_t n_route,
                                       const int32_t* sorted_ids, const int32_t* row_adapter,
                                       int32_t top_k, int64_t cap, void* stream);

/* Reads the MLORA_* launch-shape overrides from the environment again (they
 * are otherwise read once, at the first fold call). For measurement tools and
 * tests that change the environment within one process. Not safe while
 * another thread is inside a fold call; launches already enqueued or
 * captured in a graph keep the shapes they were made with. */
void mlora_reload_launch_overrides(void);

#ifdef __cplusplus
}  /* extern "C" */
#endif

#endif  /* MLORA_H_ */
