// Hash embedding store and batch key dedup on gfx950.
//
// The store follows the pages' decoupled design (marovi.ai MTGR page, 方法, training-framework
// paragraph; chenhuiyu blog "MTGR", training-system section): a compact index from key to row
// pointer plus a separate value arena, so keys can be inserted and evicted in real time and the
// index can be rebuilt larger without touching the values.
//
// Index: open addressing over lines of 8 slots {int64 key, int32 row, int32 pad} (128 bytes, one
// cache line).  A key's home line comes from a 64-bit mix of the key; lines are probed in order.
// One team of 8 lanes handles one key and reads a whole line with one 16-byte load per lane.  A
// new key goes to the first empty slot of the first line (in probe order) that is not full, so a
// lookup may stop at the first line holding an empty slot.  Slots move only from empty to a key
// (claim, compare-and-swap on the key) and from a key to a tombstone (evict); a tombstone is never
// reused until the index is rebuilt.  So two teams inserting the same key always contend for the
// same slot, and the loser finds the winner's key.
//
// Arena: a stack of free rows, the step each row was last used, and the values [rows][dim].
//
// Insert runs in three launches so that no thread ever waits for another thread's write inside
// one launch: claim (find or claim a slot per key), assign (each claimed slot pops a free row and
// initialises it; with no row left the slot becomes a tombstone), resolve (every occurrence reads
// its key's row).  The dedup of a batch uses the same claim step on a scratch index and numbers
// the distinct keys in claim order.
#include <algorithm>

#include "kernels.h"

namespace mtgr {

namespace {

constexpr int64_t kEmpty = -1;
constexpr int64_t kTomb = -2;
constexpr int kTeam = 8;            // lanes per key = slots per line

struct Slot {
  int64_t key;
  int32_t row;
  int32_t pad;
};
static_assert(sizeof(Slot) == 16, "slot layout");

struct IndexHeader {                // at the start of the index memory (256 bytes reserved)
  unsigned long long live;
  unsigned long long tombstones;
  unsigned long long dropped;       // entries a rebuild could not place
};
struct ArenaHeader {                // at the start of the arena memory (256 bytes reserved)
  int32_t free_top;                 // number of rows on the free stack
  int32_t failed;                   // insert occurrences that got no row (since init)
};

// MurmurHash3's 64-bit finaliser (Appleby, public domain): a bijective mix of all key bits.
__device__ __forceinline__ uint64_t mix64(uint64_t k) {
  k ^= k >> 33;
  k *= 0xff51afd7ed558ccdULL;
  k ^= k >> 33;
  k *= 0xc4ceb9fe1a85ec53ULL;
  k ^= k >> 33;
  return k;
}

__device__ __forceinline__ uint32_t team_ballot(bool p, int lane) {
  return (uint32_t)((__ballot(p) >> (lane & ~(kTeam - 1))) & 0xFFu);
}

// agent-coherent load of a slot key (the claim step reads lines other teams are writing)
__device__ __forceinline__ int64_t load_key_coherent(const Slot* s) {
  return __hip_atomic_load(&s->key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct View {
  IndexHeader* ih;
  Slot* slots;
  int64_t lmask;                    // lines - 1
  ArenaHeader* ah;
  int32_t* free_stack;
  int32_t* last_seen;
  char* values;
  int32_t rows;
  int32_t row_bytes;
};

// Find or claim the slot of `key` (team-uniform).  Returns the slot index, with bit 62 set when
// this team claimed it, or -1 when the index has no room.  Keys must be >= 0.
__device__ int64_t claim(const View& v, int64_t key, int lane) {
  const int sub = lane & (kTeam - 1);
  int64_t line = (int64_t)(mix64((uint64_t)key) >> 3) & v.lmask;
  for (int64_t probe = 0; probe <= v.lmask; ++probe) {
    Slot* ls = v.slots + line * kTeam;
    // A plain (cached) read that shows the key is conclusive -- slots only ever gain keys during
    // a claim -- and keeps repeated keys of a batch off the coherent path.
    const uint32_t hit = team_ballot(ls[sub].key == key, lane);
    if (hit) return line * kTeam + (__ffs(hit) - 1);
    for (;;) {
      const int64_t k = load_key_coherent(ls + sub);
      const uint32_t m = team_ballot(k == key, lane);
      if (m) return line * kTeam + (__ffs(m) - 1);
      const uint32_t e = team_ballot(k == kEmpty, lane);
      if (!e) break;                                   // full line: next one
      const int first = __ffs(e) - 1;
      int64_t old = 0;
      if (sub == first) {
        unsigned long long* p = reinterpret_cast<unsigned long long*>(&ls[first].key);
        old = (int64_t)atomicCAS(p, (unsigned long long)kEmpty, (unsigned long long)key);
      }
      old = __shfl(old, (lane & ~(kTeam - 1)) + first, kWave);
      if (old == kEmpty) return (line * kTeam + first) | (1LL << 62);
      if (old == key) return line * kTeam + first;
      // another key took the slot: read the line again
    }
    line = (line + 1) & v.lmask;
  }
  return -1;
}

// Slot index of `key`, or -1 (no concurrent writers: plain loads), probing from line `line` on,
// `probe0` lines of the sequence already seen.
__device__ int64_t find_from(const View& v, int64_t key, int64_t line, int64_t probe0, int lane) {
  const int sub = lane & (kTeam - 1);
  for (int64_t probe = probe0; probe <= v.lmask; ++probe) {
    const int64_t k = v.slots[line * kTeam + sub].key;
    const uint32_t m = team_ballot(k == key, lane);
    if (m) return line * kTeam + (__ffs(m) - 1);
    if (team_ballot(k == kEmpty, lane)) return -1;
    line = (line + 1) & v.lmask;
  }
  return -1;
}

__device__ __forceinline__ int64_t home_line(const View& v, int64_t key) {
  return (int64_t)(mix64((uint64_t)key) >> 3) & v.lmask;
}

// Slot index of `key`, or -1 (no concurrent writers: plain loads).
__device__ int64_t find(const View& v, int64_t key, int lane) {
  const int sub = lane & (kTeam - 1);
  int64_t line = home_line(v, key);
  for (int64_t probe = 0; probe <= v.lmask; ++probe) {
    const int64_t k = v.slots[line * kTeam + sub].key;
    const uint32_t m = team_ballot(k == key, lane);
    if (m) return line * kTeam + (__ffs(m) - 1);
    if (team_ballot(k == kEmpty, lane)) return -1;
    line = (line + 1) & v.lmask;
  }
  return -1;
}

// copy one value row (row_bytes, a multiple of 16) by the 8 lanes of a team; src NULL -> zeros
__device__ __forceinline__ void team_copy(char* dst, const char* src, int row_bytes, int sub) {
  for (int c = sub * 16; c < row_bytes; c += kTeam * 16) {
    uint4 v = src ? *reinterpret_cast<const uint4*>(src + c) : make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(dst + c) = v;
  }
}

inline unsigned team_grid(int64_t n) {
  const int64_t blocks = (n * kTeam + 255) / 256;
  return (unsigned)std::max<int64_t>(1, std::min<int64_t>(blocks, 65536));
}

// ---- kernels ------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_index_init(Slot* slots, int64_t nslots, IndexHeader* ih) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nslots; i += stride) {
    slots[i].key = kEmpty;
    slots[i].row = -1;
    slots[i].pad = 0;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) { ih->live = 0; ih->tombstones = 0; ih->dropped = 0; }
}

__global__ __launch_bounds__(256) void k_arena_init(ArenaHeader* ah, int32_t* free_stack, int32_t* last_seen,
                                                    int32_t rows) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < rows; i += stride) {
    free_stack[i] = rows - 1 - (int32_t)i;     // popped from the top: rows 0, 1, 2, ...
    last_seen[i] = 0;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) { ah->free_top = rows; ah->failed = 0; }
}

__global__ __launch_bounds__(256) void k_claim(View v, int64_t n, const int64_t* __restrict__ keys,
                                               int64_t* __restrict__ res) {
  const int lane = threadIdx.x & 63;
  const int64_t team = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kTeam;
  const int64_t teams = (int64_t)gridDim.x * blockDim.x / kTeam;
  for (int64_t i = team; i < n; i += teams) {
    const int64_t key = keys[i];
    const int64_t r = key >= 0 ? claim(v, key, lane) : -1;
    if ((lane & (kTeam - 1)) == 0) res[i] = r;
  }
}

// Claimed slots take a free row and initialise it; with none left the slot becomes a tombstone.
// A workgroup takes a chunk of kAssignKeys occurrences (a wavefront a quarter of it, in order):
// it counts the chunk's claimants, pops that many rows with one atomic on the stack top, and
// gives each claimant the row below the returned top by its rank within the chunk.  One atomic
// per 2048 occurrences, instead of one per wavefront step, keeps the stack top from serialising
// a large insert.
constexpr int kAssignSteps = 64;                       // team steps per wavefront and chunk
constexpr int kAssignKeys = 4 * kTeam * kAssignSteps;  // occurrences per workgroup chunk (2048)
__global__ __launch_bounds__(256) void k_assign(View v, int64_t n, int64_t* __restrict__ res,
                                                const char* __restrict__ init, int32_t step) {
  __shared__ int s_cnt[4];
  __shared__ int32_t s_top;
  const int lane = threadIdx.x & 63, sub = lane & (kTeam - 1), w = threadIdx.x >> 6;
  const int64_t nchunks = (n + kAssignKeys - 1) / kAssignKeys;
  for (int64_t chunk = blockIdx.x; chunk < nchunks; chunk += gridDim.x) {   // block-uniform
    const int64_t wave0 = chunk * kAssignKeys + (int64_t)w * kTeam * kAssignSteps;
    auto claimant = [&](int it, int64_t& i, int64_t& r) {
      i = wave0 + (int64_t)it * kTeam + (lane >> 3);
      r = (sub == 0 && i < n) ? res[i] : -1;
      return r >= 0 && (r & (1LL << 62));
    };
    // this wavefront's claimants, then the chunk's pop
    int cnt = 0;
    for (int it = 0; it < kAssignSteps; ++it) {
      int64_t i, r;
      cnt += __popcll(__ballot(claimant(it, i, r)));
    }
    if (lane == 0) s_cnt[w] = cnt;
    __syncthreads();
    if (threadIdx.x == 0) {
      const int total = s_cnt[0] + s_cnt[1] + s_cnt[2] + s_cnt[3];
      s_top = total ? atomicSub(&v.ah->free_top, total) : 0;
    }
    __syncthreads();
    int rank0 = 0;                                     // claimants of the earlier wavefronts
    for (int k = 0; k < w; ++k) rank0 += s_cnt[k];
    const int32_t top = s_top;
    int ok_n = 0, bad_n = 0;
    for (int it = 0; it < kAssignSteps; ++it) {
      int64_t i, r;
      const bool want = claimant(it, i, r);
      const unsigned long long mask = __ballot(want);
      int32_t row = -1;
      bool ok = false, bad = false;
      if (want) {
        const int64_t slot = r & ((1LL << 62) - 1);
        const int32_t t = top - (rank0 + __popcll(mask & ((1ULL << lane) - 1)));   // this claimant's stack height
        if (t >= 1) {
          row = v.free_stack[t - 1];
          v.slots[slot].row = row;
          v.last_seen[row] = step;
          ok = true;
        } else {
          v.slots[slot].key = kTomb;
          bad = true;
        }
      }
      rank0 += __popcll(mask);
      ok_n += __popcll(__ballot(ok));
      bad_n += __popcll(__ballot(bad));
      row = __shfl(row, lane & ~(kTeam - 1), kWave);
      if (row >= 0)
        team_copy(v.values + (int64_t)row * v.row_bytes, init ? init + i * v.row_bytes : nullptr, v.row_bytes, sub);
    }
    if (lane == 0) {
      if (ok_n) atomicAdd(&v.ih->live, (unsigned long long)ok_n);
      if (bad_n) atomicAdd(&v.ih->tombstones, (unsigned long long)bad_n);
    }
    __syncthreads();                                   // s_cnt and s_top are reused by the next chunk
  }
}

// every occurrence reads its key's row; failures are counted per occurrence
__global__ __launch_bounds__(256) void k_resolve(View v, int64_t n, const int64_t* __restrict__ res,
                                                 int32_t* __restrict__ rows_out, int32_t step) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  if (blockIdx.x == 0 && threadIdx.x == 0 && v.ah->free_top < 0) v.ah->free_top = 0;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const int64_t r = res[i];
    int32_t row = -1;
    if (r >= 0) {
      const int64_t slot = r & ((1LL << 62) - 1);
      if (v.slots[slot].key != kTomb) row = v.slots[slot].row;
    }
    if (row >= 0) v.last_seen[row] = step;
    else atomicAdd(&v.ah->failed, 1);
    if (rows_out) rows_out[i] = row;
  }
}

// Each team looks up two keys per iteration (i and i + teams) and requests the two keys' index
// lines, slot rows and value rows side by side, so it has two dependent chains of loads in flight.
__global__ __launch_bounds__(256) void k_lookup(View v, int64_t n, const int64_t* __restrict__ keys, int32_t step,
                                                char* __restrict__ out, int32_t* __restrict__ rows_out,
                                                const int64_t* __restrict__ n_dev) {
  const int lane = threadIdx.x & 63, sub = lane & (kTeam - 1);
  if (n_dev) n = min(n, *n_dev);
  const int64_t team = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kTeam;
  const int64_t teams = (int64_t)gridDim.x * blockDim.x / kTeam;
  for (int64_t i0 = team; i0 < n; i0 += 2 * teams) {
    const int64_t i1 = i0 + teams;
    const bool has1 = i1 < n;
    const int64_t key0 = keys[i0];
    const int64_t key1 = has1 ? keys[i1] : kEmpty;
    // first probe of both keys' sequences
    const int64_t line0 = key0 >= 0 ? home_line(v, key0) : 0;
    const int64_t line1 = key1 >= 0 ? home_line(v, key1) : 0;
    const int64_t k0 = key0 >= 0 ? v.slots[line0 * kTeam + sub].key : kEmpty;
    const int64_t k1 = key1 >= 0 ? v.slots[line1 * kTeam + sub].key : kEmpty;
    const uint32_t m0 = team_ballot(key0 >= 0 && k0 == key0, lane), e0 = team_ballot(k0 == kEmpty, lane);
    const uint32_t m1 = team_ballot(key1 >= 0 && k1 == key1, lane), e1 = team_ballot(k1 == kEmpty, lane);
    int64_t slot0 = m0 ? line0 * kTeam + (__ffs(m0) - 1) : -1;
    int64_t slot1 = m1 ? line1 * kTeam + (__ffs(m1) - 1) : -1;
    // a full home line without the key: keep probing (rare at the store's load factors)
    if (key0 >= 0 && !m0 && !e0) slot0 = find_from(v, key0, (line0 + 1) & v.lmask, 1, lane);
    if (key1 >= 0 && !m1 && !e1) slot1 = find_from(v, key1, (line1 + 1) & v.lmask, 1, lane);
    const int32_t row0 = slot0 >= 0 ? v.slots[slot0].row : -1;
    const int32_t row1 = slot1 >= 0 ? v.slots[slot1].row : -1;
    if (out) {
      const char* src0 = row0 >= 0 ? v.values + (int64_t)row0 * v.row_bytes : nullptr;
      const char* src1 = row1 >= 0 ? v.values + (int64_t)row1 * v.row_bytes : nullptr;
      char* dst0 = out + i0 * v.row_bytes;
      char* dst1 = out + i1 * v.row_bytes;
      for (int c = sub * 16; c < v.row_bytes; c += kTeam * 16) {
        const uint4 a = src0 ? *reinterpret_cast<const uint4*>(src0 + c) : make_uint4(0, 0, 0, 0);
        const uint4 b = (has1 && src1) ? *reinterpret_cast<const uint4*>(src1 + c) : make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(dst0 + c) = a;
        if (has1) *reinterpret_cast<uint4*>(dst1 + c) = b;
      }
    }
    if (sub == 0) {
      if (rows_out) {
        rows_out[i0] = row0;
        if (has1) rows_out[i1] = row1;
      }
      if (step >= 0) {
        if (row0 >= 0) v.last_seen[row0] = step;
        if (has1 && row1 >= 0) v.last_seen[row1] = step;
      }
    }
  }
}

// Evict the key at `slot` (compare-and-swap to a tombstone; one winner among duplicates) and push
// the winners' rows on the free stack: one atomic on the stack top per wavefront.  Called by every
// lane of the wavefront (want = false where there is nothing to evict).
__device__ __forceinline__ void evict_slots(View& v, bool want, int64_t slot, int64_t key, int lane) {
  bool won = false;
  int32_t row = -1;
  if (want) {
    unsigned long long* p = reinterpret_cast<unsigned long long*>(&v.slots[slot].key);
    won = (int64_t)atomicCAS(p, (unsigned long long)key, (unsigned long long)kTomb) == key;
    if (won) row = v.slots[slot].row;
  }
  const unsigned long long mask = __ballot(won);
  if (!mask) return;
  const int leader = __ffsll((long long)mask) - 1;
  const int cnt = __popcll(mask);
  int32_t top = 0;
  if (lane == leader) {
    top = atomicAdd(&v.ah->free_top, cnt);
    atomicSub(&v.ih->live, (unsigned long long)cnt);
    atomicAdd(&v.ih->tombstones, (unsigned long long)cnt);
  }
  top = __shfl(top, leader, kWave);
  if (won) v.free_stack[top + __popcll(mask & ((1ULL << lane) - 1))] = row;
}

__global__ __launch_bounds__(256) void k_evict(View v, int64_t n, const int64_t* __restrict__ keys) {
  const int lane = threadIdx.x & 63, sub = lane & (kTeam - 1);
  const int64_t team = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kTeam;
  const int64_t teams = (int64_t)gridDim.x * blockDim.x / kTeam;
  for (int64_t base = team - (lane >> 3); base < n; base += teams) {   // wave-uniform trip count
    const int64_t i = base + (lane >> 3);
    const int64_t key = i < n ? keys[i] : -1;
    const int64_t slot = key >= 0 ? find(v, key, lane) : -1;
    evict_slots(v, sub == 0 && slot >= 0, slot, key, lane);
  }
}

__global__ __launch_bounds__(256) void k_evict_older(View v, int64_t nslots, int32_t threshold) {
  const int lane = threadIdx.x & 63;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t base = (int64_t)blockIdx.x * blockDim.x + threadIdx.x - lane; base < nslots; base += stride) {
    const int64_t s = base + lane;
    bool want = false;
    int64_t key = -1;
    if (s < nslots) {
      key = v.slots[s].key;
      if (key >= 0) {
        const int32_t row = v.slots[s].row;
        want = row >= 0 && v.last_seen[row] < threshold;
      }
    }
    evict_slots(v, want, s, key, lane);
  }
}

// live entries of src re-indexed into dst (dst initialised; src keys are distinct)
__global__ __launch_bounds__(256) void k_rebuild(View src, int64_t nslots, View dst) {
  const int lane = threadIdx.x & 63, sub = lane & (kTeam - 1);
  const int64_t team = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kTeam;
  const int64_t teams = (int64_t)gridDim.x * blockDim.x / kTeam;
  for (int64_t s = team; s < nslots; s += teams) {
    const int64_t key = src.slots[s].key;
    if (key < 0) continue;                                   // team-uniform
    const int64_t r = claim(dst, key, lane);
    if (sub == 0 && r >= 0) {
      dst.slots[r & ((1LL << 62) - 1)].row = src.slots[s].row;
      atomicAdd(&dst.ih->live, 1ULL);
    } else if (sub == 0) {
      atomicAdd(&dst.ih->dropped, 1ULL);
    }
  }
}

// ---- dedup ---------------------------------------------------------------------------------
// Claim on a scratch index: res[i] = the slot of keys[i], bit 62 set where this occurrence's team
// claimed it (the key's first claimant).
__global__ __launch_bounds__(256) void k_dedup_claim(View v, int64_t n, const int64_t* __restrict__ keys,
                                                     int64_t* __restrict__ res) {
  const int lane = threadIdx.x & 63, sub = lane & (kTeam - 1);
  const int64_t team = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kTeam;
  const int64_t teams = (int64_t)gridDim.x * blockDim.x / kTeam;
  const int64_t first_of_wave = team - (lane >> 3);
  for (int64_t base = first_of_wave; base < n; base += teams) {   // wave-uniform trip count
    const int64_t i = base + (lane >> 3);
    const int64_t key = i < n ? keys[i] : -1;
    const int64_t r = key >= 0 ? claim(v, key, lane) : -1;   // negative keys are not keys
    if (sub == 0 && i < n) res[i] = r;
  }
}

// Number the claimed keys: a workgroup takes a chunk of kAssignKeys occurrences, counts its
// claimants, takes that many ids with one atomic on the count and gives them out in chunk order;
// the id goes to the key's slot and the key to unique[id].
__global__ __launch_bounds__(256) void k_dedup_number(View v, int64_t n, const int64_t* __restrict__ keys,
                                                      const int64_t* __restrict__ res, int64_t* __restrict__ uniq,
                                                      unsigned long long* __restrict__ count) {
  __shared__ int s_cnt[4];
  __shared__ unsigned long long s_base;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t nchunks = (n + kAssignKeys - 1) / kAssignKeys;
  constexpr int kPerWave = kAssignKeys / 4;
  for (int64_t chunk = blockIdx.x; chunk < nchunks; chunk += gridDim.x) {   // block-uniform
    const int64_t wave0 = chunk * kAssignKeys + (int64_t)w * kPerWave;
    int cnt = 0;
    for (int it = 0; it < kPerWave; it += 64) {
      const int64_t i = wave0 + it + lane;
      const int64_t r = i < n ? res[i] : -1;
      cnt += __popcll(__ballot(r >= 0 && (r & (1LL << 62))));
    }
    if (lane == 0) s_cnt[w] = cnt;
    __syncthreads();
    if (threadIdx.x == 0) {
      const int total = s_cnt[0] + s_cnt[1] + s_cnt[2] + s_cnt[3];
      s_base = total ? atomicAdd(count, (unsigned long long)total) : 0ULL;
    }
    __syncthreads();
    int64_t id = (int64_t)s_base;
    for (int k = 0; k < w; ++k) id += s_cnt[k];
    for (int it = 0; it < kPerWave; it += 64) {
      const int64_t i = wave0 + it + lane;
      const int64_t r = i < n ? res[i] : -1;
      const bool fresh = r >= 0 && (r & (1LL << 62));
      const unsigned long long mask = __ballot(fresh);
      if (fresh) {
        const int64_t my = id + __popcll(mask & ((1ULL << lane) - 1));
        v.slots[r & ((1LL << 62) - 1)].row = (int32_t)my;
        uniq[my] = keys[i];
      }
      id += __popcll(mask);
    }
    __syncthreads();                                   // s_cnt and s_base are reused by the next chunk
  }
}

__global__ __launch_bounds__(256) void k_dedup_inverse(View v, int64_t n, const int64_t* __restrict__ res,
                                                       int64_t* __restrict__ inverse) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const int64_t r = res[i];
    inverse[i] = r >= 0 ? (int64_t)v.slots[r & ((1LL << 62) - 1)].row : -1;
  }
}

__global__ void k_count_reset(unsigned long long* count) { *count = 0; }

inline unsigned ew(int64_t n) { return (unsigned)std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 65536)); }

View make_view(const HashDesc& h) {
  View v{};
  v.ih = reinterpret_cast<IndexHeader*>(h.index_mem);
  v.slots = reinterpret_cast<Slot*>(static_cast<char*>(h.index_mem) + kHashHeaderBytes);
  v.lmask = h.index_cap / kTeam - 1;
  if (h.arena_mem) {
    char* a = static_cast<char*>(h.arena_mem);
    v.ah = reinterpret_cast<ArenaHeader*>(a);
    v.free_stack = reinterpret_cast<int32_t*>(a + kHashHeaderBytes);
    v.last_seen = reinterpret_cast<int32_t*>(a + kHashHeaderBytes + hash_align((size_t)h.rows * 4));
    v.values = a + kHashHeaderBytes + 2 * hash_align((size_t)h.rows * 4);
  }
  v.rows = h.rows;
  v.row_bytes = h.row_bytes;
  return v;
}

}  // namespace

hipError_t launch_hash_init(const HashDesc& h, bool index, bool arena, hipStream_t s) {
  View v = make_view(h);
  if (index) k_index_init<<<ew(h.index_cap), 256, 0, s>>>(v.slots, h.index_cap, v.ih);
  if (arena) k_arena_init<<<ew(h.rows), 256, 0, s>>>(v.ah, v.free_stack, v.last_seen, h.rows);
  return hipGetLastError();
}

hipError_t launch_hash_insert(const HashDesc& h, int64_t n, const int64_t* keys, const void* init, int32_t step,
                              int32_t* rows_out, int64_t* res, hipStream_t s) {
  if (n == 0) return hipSuccess;
  View v = make_view(h);
  k_claim<<<team_grid(n), 256, 0, s>>>(v, n, keys, res);
  k_assign<<<(unsigned)std::min<int64_t>((n + kAssignKeys - 1) / kAssignKeys, 65536), 256, 0, s>>>(
      v, n, res, static_cast<const char*>(init), step);
  k_resolve<<<ew(n), 256, 0, s>>>(v, n, res, rows_out, step);
  return hipGetLastError();
}

hipError_t launch_hash_lookup(const HashDesc& h, int64_t n, const int64_t* keys, int32_t step, void* out,
                              int32_t* rows_out, hipStream_t s, const int64_t* n_dev) {
  if (n == 0) return hipSuccess;
  k_lookup<<<team_grid(n), 256, 0, s>>>(make_view(h), n, keys, step, static_cast<char*>(out), rows_out, n_dev);
  return hipGetLastError();
}

hipError_t launch_hash_evict(const HashDesc& h, int64_t n, const int64_t* keys, hipStream_t s) {
  if (n == 0) return hipSuccess;
  k_evict<<<team_grid(n), 256, 0, s>>>(make_view(h), n, keys);
  return hipGetLastError();
}

hipError_t launch_hash_evict_older(const HashDesc& h, int32_t threshold, hipStream_t s) {
  k_evict_older<<<ew(h.index_cap), 256, 0, s>>>(make_view(h), h.index_cap, threshold);
  return hipGetLastError();
}

hipError_t launch_hash_rebuild(const HashDesc& src, const HashDesc& dst, hipStream_t s) {
  View d = make_view(dst);
  k_index_init<<<ew(dst.index_cap), 256, 0, s>>>(d.slots, dst.index_cap, d.ih);
  k_rebuild<<<team_grid(src.index_cap), 256, 0, s>>>(make_view(src), src.index_cap, d);
  return hipGetLastError();
}

hipError_t launch_dedup(int64_t n, const int64_t* keys, const HashDesc& scratch, int64_t* res, int64_t* uniq,
                        int64_t* inverse, unsigned long long* count, hipStream_t s) {
  View v = make_view(scratch);
  k_index_init<<<ew(scratch.index_cap), 256, 0, s>>>(v.slots, scratch.index_cap, v.ih);
  k_count_reset<<<1, 1, 0, s>>>(count);
  if (n == 0) return hipGetLastError();
  k_dedup_claim<<<team_grid(n), 256, 0, s>>>(v, n, keys, res);
  k_dedup_number<<<(unsigned)std::min<int64_t>((n + kAssignKeys - 1) / kAssignKeys, 65536), 256, 0, s>>>(
      v, n, keys, res, uniq, count);
  k_dedup_inverse<<<ew(n), 256, 0, s>>>(v, n, res, inverse);
  return hipGetLastError();
}

}  // namespace mtgr
