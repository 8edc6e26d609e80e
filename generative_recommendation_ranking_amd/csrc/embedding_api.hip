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

// ---- tokenizer --------------------------------------------------------------------------------
struct TokPlan {
  size_t flags = 0, cnt = 0, goff = 0, keys = 0, dedup = 0, uniq = 0, inverse = 0, ucount = 0, uvals = 0;
  size_t pos = 0, rowmap = 0, feat = 0, hid = 0, y = 0, total = 0;
  bool direct = false;   // the second GEMM writes token rows directly (x fits one 31-bit range)
  size_t feat_off[4] = {0, 0, 0, 0};
  int64_t row0[4] = {0, 0, 0, 0};
  int64_t dedup_cap = 0;
};

TokPlan tok_plan(const mtgr_tokenizer_params* p, const mtgr_batch* b, int e, const int64_t* gc) {
  TokPlan pl;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off += hash_align(bytes);
    return at;
  };
  const int64_t T = b->num_tokens, B = b->num_users;
  const int64_t n = T * p->max_fields;
  pl.flags = take(4);
  pl.cnt = take((size_t)B * 4 * 8);
  pl.goff = take((size_t)4 * (B + 1) * 8);
  pl.keys = take((size_t)n * 8);
  pl.dedup_cap = dedup_cap(n);
  pl.dedup = take(index_bytes(pl.dedup_cap) + (size_t)std::max<int64_t>(n, 1) * 8);
  pl.uniq = take((size_t)n * 8);
  pl.inverse = take((size_t)n * 8);
  pl.ucount = take(8);
  pl.uvals = take((size_t)n * e * 2);
  pl.pos = take((size_t)T * 8);
  pl.direct = T * (int64_t)p->d_model * 4 < (int64_t(1) << 31);
  pl.rowmap = take(pl.direct ? (size_t)T * 4 : 0);
  size_t feat_bytes = 0;
  int64_t r0 = 0;
  for (int g = 0; g < 4; ++g) {
    pl.feat_off[g] = feat_bytes;
    feat_bytes += hash_align((size_t)gc[g] * p->num_fields[g] * e * 2);
    pl.row0[g] = r0;
    r0 += gc[g];
  }
  pl.feat = take(feat_bytes);
  pl.hid = take((size_t)T * p->d_model * 2);
  pl.y = take(pl.direct ? 0 : (size_t)T * p->d_model * 4);
  pl.total = off;
  return pl;
}

mtgr_status check_tok(const mtgr_tokenizer_params* p, const mtgr_batch* b, const mtgr_hash_table* store,
                      const int64_t* gc) {
  if (!p || !b || !store || !gc) return MTGR_ERR_NULL_ARG;
  mtgr_status st = check_table(store);
  if (st != MTGR_OK) return st;
  if (store->dtype != MTGR_BF16) return MTGR_ERR_UNSUPPORTED;
  if (b->num_users < 0 || b->num_tokens < 0) return MTGR_ERR_BAD_BATCH;
  if (b->num_users > 0 && (!b->offsets_host || !b->offsets)) return MTGR_ERR_NULL_ARG;
  if (b->num_users > 0) {
    if (b->offsets_host[0] != 0 || b->offsets_host[b->num_users] != b->num_tokens) return MTGR_ERR_BAD_BATCH;
    for (int32_t u = 0; u < b->num_users; ++u)
      if (b->offsets_host[u + 1] < b->offsets_host[u]) return MTGR_ERR_BAD_BATCH;
  } else if (b->num_tokens != 0) {
    return MTGR_ERR_BAD_BATCH;
  }
  if (b->num_tokens > 0 && !b->group_ids) return MTGR_ERR_NULL_ARG;
  int64_t sum = 0;
  for (int g = 0; g < 4; ++g) {
    if (gc[g] < 0) return MTGR_ERR_BAD_BATCH;
    sum += gc[g];
  }
  if (sum != b->num_tokens || gc[3] != b->num_candidates) return MTGR_ERR_BAD_BATCH;
  const int d = p->d_model, e = store->dim;
  if (d < 128 || d % 64 != 0 || d > 4096) return MTGR_ERR_BAD_SHAPE;
  if (p->max_fields < 1 || p->max_fields > MTGR_TOK_MAX_FIELDS) return MTGR_ERR_BAD_SHAPE;
  for (int g = 0; g < 4; ++g) {
    const int nf = p->num_fields[g];
    if (nf < 1 || nf > p->max_fields) return MTGR_ERR_BAD_SHAPE;
    if ((nf * e) % 64 != 0 || nf * e < 128) return MTGR_ERR_BAD_SHAPE;   // the GEMM's K
    for (int f = 0; f < nf; ++f)
      if (p->field_table[g][f] < 0 || p->field_table[g][f] >= (1 << 23)) return MTGR_ERR_BAD_SHAPE;
    if (gc[g] > 0 && (!p->w1[g] || !p->w2[g])) return MTGR_ERR_NULL_ARG;
  }
  return MTGR_OK;
}

}  // namespace

extern "C" {

mtgr_status mtgr_tokenize_workspace_size(const mtgr_tokenizer_params* p, const mtgr_batch* b,
                                         const mtgr_hash_table* store, const int64_t group_counts[4],
                                         size_t* bytes) {
  if (!bytes) return MTGR_ERR_NULL_ARG;
  mtgr_status st = check_tok(p, b, store, group_counts);
  if (st != MTGR_OK) return st;
  *bytes = tok_plan(p, b, store->dim, group_counts).total;
  return MTGR_OK;
}

mtgr_status mtgr_tokenize(const mtgr_tokenizer_params* p, const mtgr_batch* b, const int64_t group_counts[4],
                          const int64_t* field_ids, const mtgr_hash_table* store, int32_t step, float* x_out,
                          int32_t* flags_out, void* ws, size_t ws_bytes, void* stream) {
  mtgr_status st = check_tok(p, b, store, group_counts);
  if (st != MTGR_OK) return st;
  const int64_t T = b->num_tokens;
  if (T > 0 && (!field_ids || !x_out)) return MTGR_ERR_NULL_ARG;
  const int e = store->dim, d = p->d_model, fmax = p->max_fields;
  const TokPlan pl = tok_plan(p, b, e, group_counts);
  if (!ws || ws_bytes < pl.total) return MTGR_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  int32_t* flags = flags_out ? flags_out : reinterpret_cast<int32_t*>(w + pl.flags);
  TokFields tf{};
  for (int g = 0; g < 4; ++g) {
    tf.nfields[g] = p->num_fields[g];
    for (int f = 0; f < MTGR_TOK_MAX_FIELDS; ++f) tf.table[g][f] = f < p->num_fields[g] ? p->field_table[g][f] : 0;
  }
  int64_t* cnt = reinterpret_cast<int64_t*>(w + pl.cnt);
  int64_t* goff = reinterpret_cast<int64_t*>(w + pl.goff);
  int64_t* keys = reinterpret_cast<int64_t*>(w + pl.keys);
  int64_t* uniq = reinterpret_cast<int64_t*>(w + pl.uniq);
  int64_t* inverse = reinterpret_cast<int64_t*>(w + pl.inverse);
  int64_t* ucount = reinterpret_cast<int64_t*>(w + pl.ucount);
  bf16* uvals = reinterpret_cast<bf16*>(w + pl.uvals);
  int64_t* pos = reinterpret_cast<int64_t*>(w + pl.pos);
  bf16* hid = reinterpret_cast<bf16*>(w + pl.hid);
  float* y = reinterpret_cast<float*>(w + pl.y);
  int32_t* rowmap = pl.direct ? reinterpret_cast<int32_t*>(w + pl.rowmap) : nullptr;
  const int64_t n = T * fmax;
#define TOK_TRY(x)                                      \
  do {                                                  \
    if ((x) != hipSuccess) return MTGR_ERR_HIP;         \
  } while (0)
  TOK_TRY(launch_tok_prepare(b->num_users, T, fmax, b->offsets, b->group_ids, field_ids, tf, cnt, goff, keys, flags, s));
  if (T == 0) return MTGR_OK;
  HashDesc scratch;
  scratch.index_mem = w + pl.dedup;
  scratch.index_cap = pl.dedup_cap;
  scratch.arena_mem = nullptr;
  scratch.rows = 0;
  scratch.row_bytes = 0;
  int64_t* res = reinterpret_cast<int64_t*>(w + pl.dedup + index_bytes(pl.dedup_cap));
  TOK_TRY(launch_dedup(n, keys, scratch, res, uniq, inverse, reinterpret_cast<unsigned long long*>(ucount), s));
  TOK_TRY(launch_hash_lookup(desc(store), n, uniq, step, uvals, nullptr, s, ucount));
  TokGroups tg{};
  for (int g = 0; g < 4; ++g) {
    tg.nfields[g] = p->num_fields[g];
    tg.rows[g] = group_counts[g];
    tg.row0[g] = pl.row0[g];
    tg.feat[g] = reinterpret_cast<bf16*>(w + pl.feat + pl.feat_off[g]);
  }
  TOK_TRY(launch_tok_build(T, b->num_users, fmax, e, b->offsets, b->group_ids, cnt, goff, tg, inverse, uvals, pos,
                           rowmap, flags, s));
  if (pl.direct) TOK_TRY(launch_tok_zero_unplaced(T, d, pos, x_out, s));
  for (int g = 0; g < 4; ++g) {
    const int64_t rows = group_counts[g];
    if (rows == 0) continue;
    const int K = p->num_fields[g] * e;
    TOK_TRY(launch_gemm_bf16(rows, d, K, MTGR_EPI_SILU, tg.feat[g], static_cast<const bf16*>(p->w1[g]),
                             static_cast<const bf16*>(p->b1[g]), nullptr, hid + pl.row0[g] * d, s));
    if (pl.direct)
      TOK_TRY(launch_gemm_bf16_f32out_rows(rows, d, d, hid + pl.row0[g] * d, static_cast<const bf16*>(p->w2[g]),
                                           static_cast<const bf16*>(p->b2[g]), rowmap + pl.row0[g], T, x_out, s));
    else
      TOK_TRY(launch_gemm_bf16_f32out(rows, d, d, hid + pl.row0[g] * d, static_cast<const bf16*>(p->w2[g]),
                                      static_cast<const bf16*>(p->b2[g]), y + pl.row0[g] * d, s));
  }
  if (!pl.direct) TOK_TRY(launch_tok_scatter(T, d, pos, y, x_out, s));
#undef TOK_TRY
  return MTGR_OK;
}

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
