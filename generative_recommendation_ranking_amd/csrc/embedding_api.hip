// C ABI of the hash embedding store and the batch key dedup (argument checks and launches).
// The store is the pages' decoupled design -- a key-to-row index plus a separate value arena
// (marovi.ai MTGR page, 方法, training-framework paragraph); the dedup reduces a batch's keys to
// distinct ones before their lookup (same paragraph; chenhuiyu blog "MTGR", training-system
// section).  Every check runs on the host before anything is enqueued.
#include <algorithm>

#include "../../include/mtgr.h"
#include "kernels.h"

using namespace mtgr;

namespace {

inline bool pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

mtgr_status check_index_cap(int64_t cap) {
  return (pow2(cap) && cap >= 8 && cap <= (int64_t(1) << 40)) ? MTGR_OK : MTGR_ERR_BAD_SHAPE;
}

int row_bytes_of(int32_t dim, int32_t dtype) { return dim * (dtype == MTGR_BF16 ? 2 : 4); }

mtgr_status check_arena(int32_t rows, int32_t dim, int32_t dtype) {
  if (dtype != MTGR_F32 && dtype != MTGR_BF16) return MTGR_ERR_UNSUPPORTED;
  if (rows < 1 || dim < 1 || dim > 4096) return MTGR_ERR_BAD_SHAPE;
  if (row_bytes_of(dim, dtype) % 16 != 0) return MTGR_ERR_BAD_SHAPE;   // rows move in 16-byte pieces
  return MTGR_OK;
}

size_t index_bytes(int64_t cap) { return kHashHeaderBytes + (size_t)cap * 16; }
size_t arena_bytes(int32_t rows, int32_t dim, int32_t dtype) {
  return kHashHeaderBytes + 2 * hash_align((size_t)rows * 4) + (size_t)rows * row_bytes_of(dim, dtype);
}

mtgr_status check_table(const mtgr_hash_table* t) {
  if (!t) return MTGR_ERR_NULL_ARG;
  mtgr_status st = check_index_cap(t->index_cap);
  if (st != MTGR_OK) return st;
  if ((st = check_arena(t->rows, t->dim, t->dtype)) != MTGR_OK) return st;
  if (!t->index_mem || !t->arena_mem) return MTGR_ERR_NULL_ARG;
  return MTGR_OK;
}

HashDesc desc(const mtgr_hash_table* t) {
  HashDesc h;
  h.index_mem = t->index_mem;
  h.index_cap = t->index_cap;
  h.arena_mem = t->arena_mem;
  h.rows = t->rows;
  h.row_bytes = row_bytes_of(t->dim, t->dtype);
  return h;
}

inline mtgr_status hs(hipError_t e) { return e == hipSuccess ? MTGR_OK : MTGR_ERR_HIP; }

int64_t dedup_cap(int64_t n) {
  int64_t cap = 16;
  while (cap < 2 * n) cap <<= 1;
  return cap;
}

}  // namespace

extern "C" {

mtgr_status mtgr_hash_index_bytes(int64_t index_cap, size_t* bytes) {
  if (!bytes) return MTGR_ERR_NULL_ARG;
  mtgr_status st = check_index_cap(index_cap);
  if (st != MTGR_OK) return st;
  *bytes = index_bytes(index_cap);
  return MTGR_OK;
}

mtgr_status mtgr_hash_arena_bytes(int32_t rows, int32_t dim, int32_t dtype, size_t* bytes) {
  if (!bytes) return MTGR_ERR_NULL_ARG;
  mtgr_status st = check_arena(rows, dim, dtype);
  if (st != MTGR_OK) return st;
  *bytes = arena_bytes(rows, dim, dtype);
  return MTGR_OK;
}

mtgr_status mtgr_hash_init(const mtgr_hash_table* t, void* stream) {
  mtgr_status st = check_table(t);
  if (st != MTGR_OK) return st;
  return hs(launch_hash_init(desc(t), true, true, static_cast<hipStream_t>(stream)));
}

mtgr_status mtgr_hash_insert_workspace_size(int64_t n, size_t* bytes) {
  if (!bytes) return MTGR_ERR_NULL_ARG;
  if (n < 0) return MTGR_ERR_BAD_SHAPE;
  *bytes = (size_t)std::max<int64_t>(n, 1) * 8;
  return MTGR_OK;
}

mtgr_status mtgr_hash_insert(const mtgr_hash_table* t, int64_t n, const int64_t* keys, const void* init_values,
                             int32_t step, int32_t* rows_out, void* ws, size_t ws_bytes, void* stream) {
  mtgr_status st = check_table(t);
  if (st != MTGR_OK) return st;
  if (n < 0) return MTGR_ERR_BAD_SHAPE;
  if (n == 0) return MTGR_OK;
  if (!keys) return MTGR_ERR_NULL_ARG;
  if (!ws || ws_bytes < (size_t)n * 8) return MTGR_ERR_WORKSPACE;
  return hs(launch_hash_insert(desc(t), n, keys, init_values, step, rows_out, static_cast<int64_t*>(ws),
                               static_cast<hipStream_t>(stream)));
}

mtgr_status mtgr_hash_lookup(const mtgr_hash_table* t, int64_t n, const int64_t* keys, int32_t step,
                             void* values_out, int32_t* rows_out, void* stream) {
  mtgr_status st = check_table(t);
  if (st != MTGR_OK) return st;
  if (n < 0) return MTGR_ERR_BAD_SHAPE;
  if (n == 0) return MTGR_OK;
  if (!keys) return MTGR_ERR_NULL_ARG;
  return hs(launch_hash_lookup(desc(t), n, keys, step, values_out, rows_out, static_cast<hipStream_t>(stream)));
}

mtgr_status mtgr_hash_evict(const mtgr_hash_table* t, int64_t n, const int64_t* keys, void* stream) {
  mtgr_status st = check_table(t);
  if (st != MTGR_OK) return st;
  if (n < 0) return MTGR_ERR_BAD_SHAPE;
  if (n == 0) return MTGR_OK;
  if (!keys) return MTGR_ERR_NULL_ARG;
  return hs(launch_hash_evict(desc(t), n, keys, static_cast<hipStream_t>(stream)));
}

mtgr_status mtgr_hash_evict_older(const mtgr_hash_table* t, int32_t step_threshold, void* stream) {
  mtgr_status st = check_table(t);
  if (st != MTGR_OK) return st;
  return hs(launch_hash_evict_older(desc(t), step_threshold, static_cast<hipStream_t>(stream)));
}

mtgr_status mtgr_hash_rebuild(const mtgr_hash_table* src, void* dst_index_mem, int64_t dst_index_cap,
                              void* stream) {
  mtgr_status st = check_table(src);
  if (st != MTGR_OK) return st;
  if ((st = check_index_cap(dst_index_cap)) != MTGR_OK) return st;
  if (!dst_index_mem) return MTGR_ERR_NULL_ARG;
  if (dst_index_mem == src->index_mem) return MTGR_ERR_BAD_SHAPE;
  HashDesc d = desc(src);
  d.index_mem = dst_index_mem;
  d.index_cap = dst_index_cap;
  return hs(launch_hash_rebuild(desc(src), d, static_cast<hipStream_t>(stream)));
}

mtgr_status mtgr_hash_get_stats(const mtgr_hash_table* t, mtgr_hash_stats* out, void* stream) {
  mtgr_status st = check_table(t);
  if (st != MTGR_OK) return st;
  if (!out) return MTGR_ERR_NULL_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  unsigned long long ih[3] = {0, 0, 0};
  int32_t ah[2] = {0, 0};
  if (hipMemcpyAsync(ih, t->index_mem, sizeof(ih), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipMemcpyAsync(ah, t->arena_mem, sizeof(ah), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return MTGR_ERR_HIP;
  out->live = (int64_t)ih[0];
  out->tombstones = (int64_t)ih[1];
  out->dropped = (int64_t)ih[2];
  out->free_rows = ah[0];
  out->failed_inserts = ah[1];
  return MTGR_OK;
}

mtgr_status mtgr_dedup_workspace_size(int64_t n, size_t* bytes) {
  if (!bytes) return MTGR_ERR_NULL_ARG;
  if (n < 0) return MTGR_ERR_BAD_SHAPE;
  *bytes = index_bytes(dedup_cap(n)) + hash_align((size_t)std::max<int64_t>(n, 1) * 8);
  return MTGR_OK;
}

mtgr_status mtgr_dedup(int64_t n, const int64_t* keys, int64_t* unique_out, int64_t* inverse_out,
                       int64_t* num_unique_out, void* ws, size_t ws_bytes, void* stream) {
  size_t need = 0;
  mtgr_status st = mtgr_dedup_workspace_size(n, &need);
  if (st != MTGR_OK) return st;
  if (!num_unique_out) return MTGR_ERR_NULL_ARG;
  if (n > 0 && (!keys || !unique_out || !inverse_out)) return MTGR_ERR_NULL_ARG;
  if (!ws || ws_bytes < need) return MTGR_ERR_WORKSPACE;
  HashDesc h;
  h.index_mem = ws;
  h.index_cap = dedup_cap(n);
  h.arena_mem = nullptr;
  h.rows = 0;
  h.row_bytes = 0;
  int64_t* res = reinterpret_cast<int64_t*>(static_cast<char*>(ws) + index_bytes(h.index_cap));
  return hs(launch_dedup(n, keys, h, res, unique_out, inverse_out,
                         reinterpret_cast<unsigned long long*>(num_unique_out), static_cast<hipStream_t>(stream)));
}

}  // extern "C"
