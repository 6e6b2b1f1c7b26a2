// C ABI of libpaged_kv.so (declared in include/paged_kv.h): host-side argument
// validation, workspace sizing and dispatch to the gfx950 launchers. Nothing
// here allocates, synchronises or keeps state; every check runs before the
// first HIP call, so invalid arguments never reach the device.

#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "paged_kv.h"
#include "pkv_device.h"
#include "pkv_debug.h"
#include "pkv_launch.h"
#include "pkv_partition.h"

namespace {

constexpr int kVersion = 100;  // 0.1.0
constexpr int64_t kMaxGrid = 0x7fffffff;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Checks common to every call: element type, block size, head geometry, pool.
int check_layout(int dtype, int block_size, int num_heads, int head_dim, int num_blocks) {
  if (dtype != PKV_F16 && dtype != PKV_BF16) return PKV_ERR_UNSUPPORTED;
  if (!pkv::supported_block_size(block_size)) return PKV_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return PKV_ERR_UNSUPPORTED;
  if (num_heads < 1 || num_blocks < 1) return PKV_ERR_SHAPE;
  // in-block element offsets are 32-bit
  if ((int64_t)num_heads * head_dim * block_size > kMaxGrid) return PKV_ERR_SHAPE;
  return PKV_OK;
}

int num_partitions(int num_seqs, int num_heads, int head_dim, int max_blocks_per_seq,
                   int block_size) {
  const int64_t tokens = (int64_t)max_blocks_per_seq * block_size;
  const int pt = pkv::decode_partition_tokens(num_seqs, num_heads, head_dim, max_blocks_per_seq,
                                              block_size);
  return (int)((tokens + pt - 1) / pt);
}

// Claim flags of the backed-up items, after the partials at a 256-byte
// boundary. Only planned item orders over 512-token partitions back items up:
// their items are long enough that a slow XCD's lag is worth a claim
// (measured on MI355X, backups in every planned order: 8 x 32K tokens 634.4
// -> 626.6 us and 256 of Exp(512) 340.3 -> 338.8 us, both 512-token
// partitions; 64 of U[128, 2048] (256-token partitions) 166.8 -> 166.6 us;
// beam search through the plain call, 128 beams over shared prompt blocks
// (256-token partitions), 113.6 -> 117.8 us per step).
size_t backup_flags_offset(size_t partial_bytes) { return (partial_bytes + 255) & ~(size_t)255; }
size_t backup_flags_bytes(int num_seqs, int num_heads, int head_dim, int max_blocks_per_seq,
                          int block_size, int parts) {
  if (!pkv::plan_fits(num_seqs, parts)) return 0;
  if (pkv::decode_partition_tokens(num_seqs, num_heads, head_dim, max_blocks_per_seq,
                                   block_size) != 512)
    return 0;
  const int hg = 64 / (head_dim / 8);
  return (size_t)pkv::backup_capacity(num_seqs, parts) * (size_t)((num_heads + hg - 1) / hg) *
         sizeof(uint32_t);
}

// Validation shared by the decode entry points. Fills *parts and *need.
int check_decode(int num_seqs, int num_heads, int head_dim, int block_size,
                 int max_blocks_per_seq, int* parts, size_t* need) {
  if (num_seqs < 0 || max_blocks_per_seq < 1) return PKV_ERR_SHAPE;
  if ((int64_t)max_blocks_per_seq * block_size > kMaxGrid) return PKV_ERR_SHAPE;
  *parts = num_partitions(num_seqs, num_heads, head_dim, max_blocks_per_seq, block_size);
  if ((int64_t)num_seqs * num_heads * (*parts) > kMaxGrid) return PKV_ERR_SHAPE;
  *need = (*parts > 1) ? pkv::decode_workspace_bytes(num_seqs, num_heads, head_dim, *parts) : 0;
  if (*need)
    *need = backup_flags_offset(*need) + backup_flags_bytes(num_seqs, num_heads, head_dim,
                                                            max_blocks_per_seq, block_size, *parts);
  return PKV_OK;
}

int check_workspace(void* ws, size_t bytes, size_t need) {
  if (need == 0) return PKV_OK;
  if (ws == nullptr || bytes < need) return PKV_ERR_WORKSPACE;
  if (!aligned16(ws)) return PKV_ERR_ALIGN;
  return PKV_OK;
}

int status_of(hipError_t e) { return e == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH; }

// With PAGED_KV_DEBUG=1: run `checks` (device checks of the call's
// data-dependent preconditions) on the stream, wait for them, and return
// PKV_ERR_DATA if one failed, before the call launches anything else.
// Otherwise nothing is launched and PKV_OK is returned.
template <typename F>
int debug_gate(hipStream_t st, F&& checks) {
  if (!pkv::debug_enabled()) return PKV_OK;
  hipError_t e = pkv::debug_reset(st);
  if (e == hipSuccess) e = checks();
  unsigned status = 0u;
  if (e == hipSuccess) e = pkv::debug_status(st, &status);
  if (e != hipSuccess) return PKV_ERR_LAUNCH;
  return status ? PKV_ERR_DATA : PKV_OK;
}

int debug_decode(const pkv::DecodeArgs& a, int num_blocks, hipStream_t st) {
  return debug_gate(st, [&] {
    return pkv::debug_check_tables(a.block_tables, a.context_lens, a.num_seqs,
                                   a.max_blocks_per_seq, a.block_size, num_blocks, 1, st);
  });
}

int prepare_decode(pkv::DecodeArgs* a, void* out, const void* query, const void* key_cache,
                   const void* value_cache, const int32_t* block_tables,
                   const int32_t* context_lens, int num_seqs, int num_heads, int head_dim,
                   int num_blocks, int block_size, int max_blocks_per_seq, float scale, int dtype,
                   void* workspace, size_t workspace_bytes) {
  int rc = check_layout(dtype, block_size, num_heads, head_dim, num_blocks);
  if (rc) return rc;
  int parts = 0;
  size_t need = 0;
  rc = check_decode(num_seqs, num_heads, head_dim, block_size, max_blocks_per_seq, &parts, &need);
  if (rc) return rc;
  if (!isfinite(scale)) return PKV_ERR_SHAPE;
  if (num_seqs == 0) return PKV_OK;  // nothing to do; empty tensors may carry NULL
  if (!out || !query || !key_cache || !value_cache || !block_tables || !context_lens)
    return PKV_ERR_NULL;
  if (!aligned16(out) || !aligned16(query) || !aligned16(key_cache) || !aligned16(value_cache) ||
      !aligned4(block_tables) || !aligned4(context_lens))
    return PKV_ERR_ALIGN;
  rc = check_workspace(workspace, workspace_bytes, need);
  if (rc) return rc;
  a->out = out;
  a->query = query;
  a->key_cache = key_cache;
  a->value_cache = value_cache;
  a->block_tables = block_tables;
  a->context_lens = context_lens;
  a->num_seqs = num_seqs;
  a->num_heads = num_heads;
  a->head_dim = head_dim;
  a->max_blocks_per_seq = max_blocks_per_seq;
  a->block_size = block_size;
  a->num_parts = parts;
  a->part_tokens = pkv::decode_partition_tokens(num_seqs, num_heads, head_dim,
                                                  max_blocks_per_seq, block_size);
  a->scale = scale;
  a->dtype = dtype;
  a->tail_parts = parts;
  a->slot_base = 0;
  a->group_start = nullptr;
  a->shared_blocks = nullptr;
  a->num_groups = 0;
  a->ws_ml = nullptr;
  a->ws_o = nullptr;
  a->ws_seq = nullptr;
  a->flags = nullptr;
  a->backup_items = 0;
  if (need) pkv::decode_workspace_split(workspace, num_seqs, num_heads, parts, &a->ws_ml, &a->ws_o);
  if (need && backup_flags_bytes(num_seqs, num_heads, head_dim, max_blocks_per_seq, block_size,
                                 parts)) {
    a->flags = reinterpret_cast<uint32_t*>(
        static_cast<char*>(workspace) +
        backup_flags_offset(pkv::decode_workspace_bytes(num_seqs, num_heads, head_dim, parts)));
    a->backup_items = pkv::backup_capacity(num_seqs, parts);
  }
  return PKV_OK;
}

// Tail partitions of the grouped call are 512 tokens whatever the table size.
// A tail (the context past the shared prefix) is usually much shorter than the
// table, and the grid is sized from the table: longer partitions leave fewer
// workgroups with nothing to do and fewer partials to merge (measured faster
// than 256 on the shared-prefix and beam-search steps at block sizes 8-32).
constexpr int kGroupedTailTokens = 512;

// Partial slots of the grouped call: shared-prefix chunks, then tail partitions.
void grouped_slots(int max_blocks_per_seq, int block_size, int* chunk_slots, int* tail_parts) {
  // shared tokens <= max_blocks_per_seq * block_size, in chunks of kSharedChunkTiles tiles of 16
  constexpr int64_t chunk_tokens = pkv::kSharedChunkTiles * pkv::kTileTokens;
  const int64_t tokens = (int64_t)max_blocks_per_seq * block_size;
  *chunk_slots = (int)((tokens + chunk_tokens - 1) / chunk_tokens);
  *tail_parts = (int)((tokens + kGroupedTailTokens - 1) / kGroupedTailTokens);
}

int check_grouped(int num_seqs, int num_heads, int head_dim, int block_size,
                  int max_blocks_per_seq, int num_groups, int* chunk_slots, int* tail_parts,
                  size_t* need) {
  if (num_seqs < 0 || max_blocks_per_seq < 1 || num_groups < 0) return PKV_ERR_SHAPE;
  if (num_seqs > 0 && num_groups < 1) return PKV_ERR_SHAPE;
  if ((int64_t)max_blocks_per_seq * block_size > kMaxGrid) return PKV_ERR_SHAPE;
  grouped_slots(max_blocks_per_seq, block_size, chunk_slots, tail_parts);
  const int64_t slots = (int64_t)*chunk_slots + *tail_parts;
  if ((int64_t)num_seqs * num_heads * slots > kMaxGrid) return PKV_ERR_SHAPE;
  if ((int64_t)num_groups * (*chunk_slots) * num_heads + (int64_t)num_seqs * num_heads * slots >
      kMaxGrid)
    return PKV_ERR_SHAPE;
  // partials, then one int32 per sequence (its shared-prefix token count)
  *need = pkv::decode_workspace_bytes(num_seqs, num_heads, head_dim, (int)slots) +
          (size_t)num_seqs * sizeof(int32_t);
  return PKV_OK;
}

// Device address under which the current device reaches [ptr, ptr + bytes):
// device memory of this device, or pinned (page-locked, mapped) host memory.
// Anything else (pageable host memory, another device's memory, a range that
// runs past its allocation) is refused with PKV_ERR_MEMORY before any launch.
int device_accessible(const void* ptr, size_t bytes, const void** dev_ptr, bool* host = nullptr) {
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, ptr) != hipSuccess) {
    (void)hipGetLastError();  // clear the sticky error of the failed query
    return PKV_ERR_MEMORY;
  }
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return PKV_ERR_MEMORY;
  if (attr.type == hipMemoryTypeDevice) {
    if (attr.device != dev) return PKV_ERR_MEMORY;
    *dev_ptr = ptr;
  } else if (attr.type == hipMemoryTypeHost) {
    if (attr.devicePointer == nullptr) return PKV_ERR_MEMORY;
    *dev_ptr = attr.devicePointer;
    if (host) *host = true;
  } else {
    return PKV_ERR_MEMORY;
  }
  hipDeviceptr_t base = nullptr;
  size_t size = 0;
  if (hipMemGetAddressRange(&base, &size, const_cast<void*>(*dev_ptr)) != hipSuccess) {
    (void)hipGetLastError();
    return PKV_ERR_MEMORY;
  }
  const uintptr_t b = reinterpret_cast<uintptr_t>(base);
  const uintptr_t p = reinterpret_cast<uintptr_t>(*dev_ptr);
  if (p < b || bytes > size || p - b > size - bytes) return PKV_ERR_MEMORY;
  return PKV_OK;
}

// Scratch of paged_attention_decode_noalloc: the split-K partials of one
// call, in a fixed device array (each GPU the library runs on holds its own
// copy until the process ends). Host code never passes the array's name to a
// kernel: it is a host-side stand-in, not a device address. The device
// address comes from hipGetSymbolAddress, once per device, with that device
// current.
static __device__ __align__(256) uint8_t scratch[PKV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, or nullptr (with the
// HIP error cleared) if it cannot be had.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int pkv_version(void) { return kVersion; }

const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "success";
    case PKV_ERR_NULL: return "a required pointer is NULL";
    case PKV_ERR_SHAPE: return "argument out of range (count, size overflow or non-finite scale)";
    case PKV_ERR_UNSUPPORTED: return "unsupported dtype, block_size or head_dim";
    case PKV_ERR_MEMORY:
      return "a buffer is not device memory of the current device or pinned host memory, "
             "or is smaller than its sizes say";
    case PKV_ERR_WORKSPACE: return "workspace missing or too small";
    case PKV_ERR_LAUNCH: return "kernel launch failed";
    case PKV_ERR_ALIGN: return "pointer not 16-byte aligned";
    case PKV_ERR_SCRATCH:
      return "the call needs more split-K scratch than paged_attention_decode_noalloc's fixed "
             "device array holds (PKV_NOALLOC_SCRATCH_BYTES); use paged_attention_decode with a "
             "workspace";
    case PKV_ERR_DATA:
      return "a data-dependent precondition does not hold (found by the PAGED_KV_DEBUG=1 "
             "device checks; nothing was launched)";
    default: return "unknown status";
  }
}

size_t paged_attention_workspace_size(int num_seqs, int num_heads, int head_dim,
                                      int max_blocks_per_seq, int block_size) {
  if (check_layout(PKV_F16, block_size, num_heads, head_dim, 1)) return 0;
  int parts = 0;
  size_t need = 0;
  if (check_decode(num_seqs, num_heads, head_dim, block_size, max_blocks_per_seq, &parts, &need))
    return 0;
  return need;
}

int paged_attention_decode_partitions(void* out, const void* query, const void* key_cache,
                                      const void* value_cache, const int32_t* block_tables,
                                      const int32_t* context_lens, int num_seqs, int num_heads,
                                      int head_dim, int num_blocks, int block_size,
                                      int max_blocks_per_seq, float scale, int dtype,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  pkv::DecodeArgs a;
  int rc = prepare_decode(&a, out, query, key_cache, value_cache, block_tables, context_lens,
                          num_seqs, num_heads, head_dim, num_blocks, block_size,
                          max_blocks_per_seq, scale, dtype, workspace, workspace_bytes);
  if (rc || num_seqs == 0) return rc;
  if ((rc = debug_decode(a, num_blocks, static_cast<hipStream_t>(stream)))) return rc;
  return status_of(pkv::launch_decode_partitions(a, static_cast<hipStream_t>(stream)));
}

int paged_attention_decode_merge(void* out, const int32_t* context_lens, int num_seqs,
                                 int num_heads, int head_dim, int block_size,
                                 int max_blocks_per_seq, int dtype, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  int rc = check_layout(dtype, block_size, num_heads, head_dim, 1);
  if (rc) return rc;
  int parts = 0;
  size_t need = 0;
  rc = check_decode(num_seqs, num_heads, head_dim, block_size, max_blocks_per_seq, &parts, &need);
  if (rc) return rc;
  if (num_seqs == 0) return PKV_OK;
  if (!out || !context_lens) return PKV_ERR_NULL;
  if (!aligned16(out) || !aligned4(context_lens)) return PKV_ERR_ALIGN;
  rc = check_workspace(workspace, workspace_bytes, need);
  if (rc) return rc;
  if (parts <= 1) return PKV_OK;  // every sequence was finished by the first launch
  pkv::DecodeArgs a = {};
  a.out = out;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.head_dim = head_dim;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.block_size = block_size;
  a.num_parts = parts;
  a.tail_parts = parts;
  a.part_tokens = pkv::decode_partition_tokens(num_seqs, num_heads, head_dim,
                                                  max_blocks_per_seq, block_size);
  a.dtype = dtype;
  pkv::decode_workspace_split(workspace, num_seqs, num_heads, parts, &a.ws_ml, &a.ws_o);
  return status_of(pkv::launch_decode_merge(a, static_cast<hipStream_t>(stream)));
}

int paged_attention_decode(void* out, const void* query, const void* key_cache,
                           const void* value_cache, const int32_t* block_tables,
                           const int32_t* context_lens, int num_seqs, int num_heads, int head_dim,
                           int num_blocks, int block_size, int max_blocks_per_seq, float scale,
                           int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  pkv::DecodeArgs a;
  int rc = prepare_decode(&a, out, query, key_cache, value_cache, block_tables, context_lens,
                          num_seqs, num_heads, head_dim, num_blocks, block_size,
                          max_blocks_per_seq, scale, dtype, workspace, workspace_bytes);
  if (rc || num_seqs == 0) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if ((rc = debug_decode(a, num_blocks, st))) return rc;
  rc = status_of(pkv::launch_decode_partitions(a, st));
  if (rc || a.num_parts <= 1) return rc;
  return status_of(pkv::launch_decode_merge(a, st));
}

int paged_attention_decode_noalloc(void* out, const void* query, const void* key_cache,
                                   const void* value_cache, const int32_t* block_tables,
                                   const int32_t* context_lens, int num_seqs, int num_heads,
                                   int head_dim, int num_blocks, int block_size,
                                   int max_blocks_per_seq, float scale, int dtype, void* stream) {
  // Host-side checks first (nothing touches the device before they pass).
  int rc = check_layout(dtype, block_size, num_heads, head_dim, num_blocks);
  if (rc) return rc;
  int parts = 0;
  size_t need = 0;
  rc = check_decode(num_seqs, num_heads, head_dim, block_size, max_blocks_per_seq, &parts, &need);
  if (rc) return rc;
  if (!isfinite(scale)) return PKV_ERR_SHAPE;
  if (need > (size_t)PKV_NOALLOC_SCRATCH_BYTES) return PKV_ERR_SCRATCH;
  if (num_seqs == 0) return PKV_OK;
  if (!out || !query || !key_cache || !value_cache || !block_tables || !context_lens)
    return PKV_ERR_NULL;
  if (!aligned16(out) || !aligned16(query) || !aligned16(key_cache) || !aligned16(value_cache) ||
      !aligned4(block_tables) || !aligned4(context_lens))
    return PKV_ERR_ALIGN;
  void* ws = nullptr;
  if (need) {
    ws = scratch_on_current_device();
    if (ws == nullptr) return PKV_ERR_LAUNCH;
  }
  return paged_attention_decode(out, query, key_cache, value_cache, block_tables, context_lens,
                                num_seqs, num_heads, head_dim, num_blocks, block_size,
                                max_blocks_per_seq, scale, dtype, ws,
                                (size_t)PKV_NOALLOC_SCRATCH_BYTES, stream);
}

size_t paged_attention_grouped_workspace_size(int num_seqs, int num_heads, int head_dim,
                                              int max_blocks_per_seq, int block_size) {
  if (check_layout(PKV_F16, block_size, num_heads, head_dim, 1)) return 0;
  int cs = 0, tp = 0;
  size_t need = 0;
  if (check_grouped(num_seqs, num_heads, head_dim, block_size, max_blocks_per_seq, 1, &cs, &tp,
                    &need))
    return 0;
  return need;
}

int paged_attention_decode_grouped(void* out, const void* query, const void* key_cache,
                                   const void* value_cache, const int32_t* block_tables,
                                   const int32_t* context_lens, const int32_t* group_start,
                                   const int32_t* shared_blocks, int num_groups, int num_seqs,
                                   int num_heads, int head_dim, int num_blocks, int block_size,
                                   int max_blocks_per_seq, float scale, int dtype,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_layout(dtype, block_size, num_heads, head_dim, num_blocks);
  if (rc) return rc;
  int chunk_slots = 0, tail_parts = 0;
  size_t need = 0;
  rc = check_grouped(num_seqs, num_heads, head_dim, block_size, max_blocks_per_seq, num_groups,
                     &chunk_slots, &tail_parts, &need);
  if (rc) return rc;
  if (!isfinite(scale)) return PKV_ERR_SHAPE;
  if (num_seqs == 0) return PKV_OK;
  if (!out || !query || !key_cache || !value_cache || !block_tables || !context_lens ||
      !group_start || !shared_blocks)
    return PKV_ERR_NULL;
  if (!aligned16(out) || !aligned16(query) || !aligned16(key_cache) || !aligned16(value_cache) ||
      !aligned4(block_tables) || !aligned4(context_lens) || !aligned4(group_start) ||
      !aligned4(shared_blocks))
    return PKV_ERR_ALIGN;
  rc = check_workspace(workspace, workspace_bytes, need);
  if (rc) return rc;
  pkv::DecodeArgs a = {};
  a.out = out;
  a.query = query;
  a.key_cache = key_cache;
  a.value_cache = value_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.head_dim = head_dim;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.block_size = block_size;
  a.part_tokens = kGroupedTailTokens;
  a.num_parts = chunk_slots + tail_parts;
  a.tail_parts = tail_parts;
  a.slot_base = chunk_slots;
  a.group_start = group_start;
  a.shared_blocks = shared_blocks;
  a.num_groups = num_groups;
  a.scale = scale;
  a.dtype = dtype;
  pkv::decode_workspace_split(workspace, num_seqs, num_heads, a.num_parts, &a.ws_ml, &a.ws_o);
  a.ws_seq = reinterpret_cast<int32_t*>(
      static_cast<char*>(workspace) +
      pkv::decode_workspace_bytes(num_seqs, num_heads, head_dim, a.num_parts));
  hipStream_t st = static_cast<hipStream_t>(stream);
  rc = debug_gate(st, [&] {
    hipError_t e = pkv::debug_check_tables(block_tables, context_lens, num_seqs,
                                           max_blocks_per_seq, block_size, num_blocks, 1, st);
    if (e != hipSuccess) return e;
    return pkv::debug_check_groups(group_start, shared_blocks, num_groups, num_seqs, block_tables,
                                   context_lens, max_blocks_per_seq, block_size, st);
  });
  if (rc) return rc;
  rc = status_of(pkv::launch_decode_grouped(a, st));
  if (rc) return rc;
  return status_of(pkv::launch_decode_merge(a, st));
}

int reshape_and_cache(const void* key, const void* value, void* key_cache, void* value_cache,
                      const int64_t* slot_mapping, int num_tokens, int num_heads, int head_dim,
                      int num_blocks, int block_size, int dtype, void* stream) {
  int rc = check_layout(dtype, block_size, num_heads, head_dim, num_blocks);
  if (rc) return rc;
  if (num_tokens < 0) return PKV_ERR_SHAPE;
  if (num_tokens == 0) return PKV_OK;  // empty tensors may carry NULL
  if (!key || !value || !key_cache || !value_cache || !slot_mapping) return PKV_ERR_NULL;
  if (!aligned16(key) || !aligned16(value) || !aligned16(key_cache) || !aligned16(value_cache) ||
      (reinterpret_cast<uintptr_t>(slot_mapping) & 7u))
    return PKV_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  rc = debug_gate(st, [&] {
    return pkv::debug_check_slots(slot_mapping, num_tokens, (int64_t)num_blocks * block_size, st);
  });
  if (rc) return rc;
  return status_of(pkv::launch_reshape_and_cache(key, value, key_cache, value_cache, slot_mapping,
                                                 num_tokens, num_heads * head_dim, st));
}

int copy_blocks(void* key_cache, void* value_cache, const int32_t* block_mapping, int num_pairs,
                int num_heads, int head_dim, int num_blocks, int block_size, int dtype,
                void* stream) {
  int rc = check_layout(dtype, block_size, num_heads, head_dim, num_blocks);
  if (rc) return rc;
  if (num_pairs < 0) return PKV_ERR_SHAPE;
  const int64_t block_elems = (int64_t)block_size * num_heads * head_dim;
  const int64_t groups = (block_elems / 8 + pkv::kCopyVecsPerGroup - 1) / pkv::kCopyVecsPerGroup;
  if ((int64_t)num_pairs * 2 * groups > kMaxGrid) return PKV_ERR_SHAPE;
  if (num_pairs == 0) return PKV_OK;  // empty tensors may carry NULL
  if (!key_cache || !value_cache || !block_mapping) return PKV_ERR_NULL;
  if (!aligned16(key_cache) || !aligned16(value_cache) || !aligned4(block_mapping))
    return PKV_ERR_ALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  rc = debug_gate(st, [&] {
    return pkv::debug_check_pairs(block_mapping, num_pairs, num_blocks, num_blocks, true, st);
  });
  if (rc) return rc;
  return status_of(pkv::launch_copy_blocks(key_cache, value_cache, key_cache, value_cache,
                                           block_mapping, num_pairs, block_elems, false, st));
}

int paged_attention_prefill(void* out, const void* query, const void* key_cache,
                            const void* value_cache, const int32_t* block_tables,
                            const int32_t* context_lens, const int32_t* query_start,
                            int num_seqs, int max_query_len, int num_heads, int head_dim,
                            int num_blocks, int block_size, int max_blocks_per_seq, float scale,
                            int dtype, void* stream) {
  int rc = check_layout(dtype, block_size, num_heads, head_dim, num_blocks);
  if (rc) return rc;
  if (num_seqs < 0 || max_query_len < 0 || max_blocks_per_seq < 1) return PKV_ERR_SHAPE;
  if ((int64_t)max_blocks_per_seq * block_size > kMaxGrid) return PKV_ERR_SHAPE;
  if (max_query_len > max_blocks_per_seq * block_size) return PKV_ERR_SHAPE;
  if (num_seqs > 65535) return PKV_ERR_SHAPE;  // grid y
  const int64_t tiles = (max_query_len + pkv::prefill_rows_per_tile() - 1) /
                        pkv::prefill_rows_per_tile();
  if (tiles * num_heads > kMaxGrid) return PKV_ERR_SHAPE;
  if (!isfinite(scale)) return PKV_ERR_SHAPE;
  if (num_seqs == 0 || max_query_len == 0) return PKV_OK;
  if (!out || !query || !key_cache || !value_cache || !block_tables || !context_lens ||
      !query_start)
    return PKV_ERR_NULL;
  if (!aligned16(out) || !aligned16(query) || !aligned16(key_cache) || !aligned16(value_cache) ||
      !aligned4(block_tables) || !aligned4(context_lens) || !aligned4(query_start))
    return PKV_ERR_ALIGN;
  pkv::PrefillArgs a = {};
  a.out = out;
  a.query = query;
  a.key_cache = key_cache;
  a.value_cache = value_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start = query_start;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.head_dim = head_dim;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.block_size = block_size;
  a.max_query_len = max_query_len;
  a.scale = scale;
  a.dtype = dtype;
  hipStream_t st = static_cast<hipStream_t>(stream);
  rc = debug_gate(st, [&] {
    hipError_t e = pkv::debug_check_tables(block_tables, context_lens, num_seqs,
                                           max_blocks_per_seq, block_size, num_blocks, 0, st);
    if (e != hipSuccess) return e;
    return pkv::debug_check_prefill(query_start, context_lens, num_seqs, max_query_len, st);
  });
  if (rc) return rc;
  return status_of(pkv::launch_prefill(a, st));
}

int swap_blocks(const void* src_key, const void* src_value, void* dst_key, void* dst_value,
                const int32_t* block_mapping, int num_pairs, int num_heads, int head_dim,
                int src_num_blocks, int dst_num_blocks, int block_size, int dtype, void* stream) {
  int rc = check_layout(dtype, block_size, num_heads, head_dim, src_num_blocks);
  if (rc) return rc;
  if (dst_num_blocks < 1) return PKV_ERR_SHAPE;
  if (num_pairs < 0) return PKV_ERR_SHAPE;
  const int64_t block_elems = (int64_t)block_size * num_heads * head_dim;
  const int64_t groups = (block_elems / 8 + pkv::kCopyVecsPerGroup - 1) / pkv::kCopyVecsPerGroup;
  if ((int64_t)num_pairs * 2 * groups > kMaxGrid) return PKV_ERR_SHAPE;
  if (num_pairs == 0) return PKV_OK;  // empty tensors may carry NULL
  if (!src_key || !src_value || !dst_key || !dst_value || !block_mapping) return PKV_ERR_NULL;
  if (!aligned16(src_key) || !aligned16(src_value) || !aligned16(dst_key) ||
      !aligned16(dst_value) || !aligned4(block_mapping))
    return PKV_ERR_ALIGN;
  const size_t block_bytes = (size_t)block_elems * sizeof(uint16_t);
  const void *sk, *sv, *dk, *dv, *bm;
  bool host_dst = false;
  if ((rc = device_accessible(src_key, block_bytes * src_num_blocks, &sk)) ||
      (rc = device_accessible(src_value, block_bytes * src_num_blocks, &sv)) ||
      (rc = device_accessible(dst_key, block_bytes * dst_num_blocks, &dk, &host_dst)) ||
      (rc = device_accessible(dst_value, block_bytes * dst_num_blocks, &dv, &host_dst)) ||
      (rc = device_accessible(block_mapping, (size_t)num_pairs * 2 * sizeof(int32_t), &bm)))
    return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  rc = debug_gate(st, [&] {
    return pkv::debug_check_pairs(static_cast<const int32_t*>(bm), num_pairs, src_num_blocks,
                                  dst_num_blocks, false, st);
  });
  if (rc) return rc;
  // The system-scope release (an L2 write-back in every workgroup) is needed
  // only when the kernel writes pinned host memory.
  return status_of(pkv::launch_copy_blocks(sk, sv, const_cast<void*>(dk), const_cast<void*>(dv),
                                           static_cast<const int32_t*>(bm), num_pairs,
                                           block_elems, host_dst, st));
}


int swap_blocks_dma(const void* src_key, const void* src_value, void* dst_key, void* dst_value,
                    const int32_t* block_mapping, int num_pairs, int num_heads, int head_dim,
                    int src_num_blocks, int dst_num_blocks, int block_size, int dtype,
                    void* stream) {
  int rc = check_layout(dtype, block_size, num_heads, head_dim, src_num_blocks);
  if (rc) return rc;
  if (dst_num_blocks < 1 || num_pairs < 0) return PKV_ERR_SHAPE;
  if (num_pairs == 0) return PKV_OK;
  if (!src_key || !src_value || !dst_key || !dst_value || !block_mapping) return PKV_ERR_NULL;
  if (!aligned16(src_key) || !aligned16(src_value) || !aligned16(dst_key) ||
      !aligned16(dst_value) || !aligned4(block_mapping))
    return PKV_ERR_ALIGN;
  // The mapping is host memory here: every id is checked before any copy.
  for (int i = 0; i < num_pairs; ++i) {
    const int32_t sb = block_mapping[2 * i], db = block_mapping[2 * i + 1];
    if (sb < 0 || sb >= src_num_blocks || db < 0 || db >= dst_num_blocks) return PKV_ERR_SHAPE;
  }
  const size_t block_bytes = (size_t)block_size * num_heads * head_dim * sizeof(uint16_t);
  const void *sk, *sv, *dk, *dv;
  if ((rc = device_accessible(src_key, block_bytes * src_num_blocks, &sk)) ||
      (rc = device_accessible(src_value, block_bytes * src_num_blocks, &sv)) ||
      (rc = device_accessible(dst_key, block_bytes * dst_num_blocks, &dk)) ||
      (rc = device_accessible(dst_value, block_bytes * dst_num_blocks, &dv)))
    return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // Runs of pairs whose source and destination ids both step by one become
  // one copy per pool.
  for (int i = 0; i < num_pairs;) {
    const int32_t s0 = block_mapping[2 * i], d0 = block_mapping[2 * i + 1];
    int n = 1;
    while (i + n < num_pairs && block_mapping[2 * (i + n)] == s0 + n &&
           block_mapping[2 * (i + n) + 1] == d0 + n)
      ++n;
    const size_t bytes = block_bytes * (size_t)n;
    const size_t so = block_bytes * (size_t)s0, doff = block_bytes * (size_t)d0;
    if (hipMemcpyAsync(static_cast<char*>(const_cast<void*>(dk)) + doff,
                       static_cast<const char*>(sk) + so, bytes, hipMemcpyDefault, st) !=
            hipSuccess ||
        hipMemcpyAsync(static_cast<char*>(const_cast<void*>(dv)) + doff,
                       static_cast<const char*>(sv) + so, bytes, hipMemcpyDefault, st) !=
            hipSuccess)
      return PKV_ERR_LAUNCH;
    i += n;
  }
  return PKV_OK;
}


int swap_blocks_staged(const void* src_key, const void* src_value, void* dst_key,
                       void* dst_value, const int32_t* block_mapping, int num_pairs,
                       int num_heads, int head_dim, int src_num_blocks, int dst_num_blocks,
                       int block_size, int dtype, void* staging, size_t staging_bytes,
                       void* stream) {
  int rc = check_layout(dtype, block_size, num_heads, head_dim, src_num_blocks);
  if (rc) return rc;
  if (dst_num_blocks < 1 || num_pairs < 0) return PKV_ERR_SHAPE;
  if (num_pairs == 0) return PKV_OK;
  if (!src_key || !src_value || !dst_key || !dst_value || !block_mapping || !staging)
    return PKV_ERR_NULL;
  if (!aligned16(src_key) || !aligned16(src_value) || !aligned16(dst_key) ||
      !aligned16(dst_value) || !aligned4(block_mapping) ||
      (reinterpret_cast<uintptr_t>(staging) & 255u))
    return PKV_ERR_ALIGN;
  for (int i = 0; i < num_pairs; ++i) {
    const int32_t sb = block_mapping[2 * i], db = block_mapping[2 * i + 1];
    if (sb < 0 || sb >= src_num_blocks || db < 0 || db >= dst_num_blocks) return PKV_ERR_SHAPE;
  }
  const size_t block_bytes = (size_t)block_size * num_heads * head_dim * sizeof(uint16_t);
  // Staging: [K slots][V slots], reused chunk by chunk.
  if (staging_bytes < 2 * block_bytes) return PKV_ERR_WORKSPACE;
  const int cap = (int)std::min<size_t>(staging_bytes / (2 * block_bytes), (size_t)num_pairs);
  const void *sk, *sv, *dk, *dv, *stg;
  bool host_dst = false;
  if ((rc = device_accessible(src_key, block_bytes * src_num_blocks, &sk)) ||
      (rc = device_accessible(src_value, block_bytes * src_num_blocks, &sv)) ||
      (rc = device_accessible(dst_key, block_bytes * dst_num_blocks, &dk, &host_dst)) ||
      (rc = device_accessible(dst_value, block_bytes * dst_num_blocks, &dv, &host_dst)) ||
      (rc = device_accessible(staging, 2 * (size_t)cap * block_bytes, &stg)))
    return rc;
  char* st_k = static_cast<char*>(const_cast<void*>(stg));
  char* st_v = st_k + (size_t)cap * block_bytes;
  hipStream_t st = static_cast<hipStream_t>(stream);
  for (int c0 = 0; c0 < num_pairs; c0 += cap) {
    const int n = std::min(cap, num_pairs - c0);
    // DMA: each run of consecutive source ids into consecutive staging slots.
    for (int i = 0; i < n;) {
      const int32_t s0 = block_mapping[2 * (c0 + i)];
      int r = 1;
      while (i + r < n && block_mapping[2 * (c0 + i + r)] == s0 + r) ++r;
      const size_t bytes = block_bytes * (size_t)r;
      const size_t so = block_bytes * (size_t)s0, to = block_bytes * (size_t)i;
      if (hipMemcpyAsync(st_k + to, static_cast<const char*>(sk) + so, bytes, hipMemcpyDefault,
                         st) != hipSuccess ||
          hipMemcpyAsync(st_v + to, static_cast<const char*>(sv) + so, bytes, hipMemcpyDefault,
                         st) != hipSuccess)
        return PKV_ERR_LAUNCH;
      i += r;
    }
    // Scatter: staging slot -> destination block, the destination ids of up
    // to kScatterIds pairs in each launch's arguments.
    for (int b0 = 0; b0 < n; b0 += pkv::kScatterIds) {
      const int nb = std::min(pkv::kScatterIds, n - b0);
      pkv::ScatterIds ids;
      for (int i = 0; i < nb; ++i) ids.dst[i] = block_mapping[2 * (c0 + b0 + i) + 1];
      rc = status_of(pkv::launch_scatter_blocks(st_k, st_v, const_cast<void*>(dk),
                                                const_cast<void*>(dv), ids, nb, b0,
                                                (int64_t)block_size * num_heads * head_dim,
                                                /*system_release=*/host_dst, st));
      if (rc) return rc;
    }
  }
  return PKV_OK;
}

}  // extern "C"
