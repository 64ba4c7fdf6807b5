// Dispatch: per-expert counts, capacity, expert-sorted permutation.
// [rkmt] "大模型MoE架构揭秘：为什么总参数≠激活参数" §2.3: each expert takes at most C
// slots; the overflow is dropped or sent to the next-best expert; [200B-5]
// "四个专家同时算，选两个会更快吗？": every selection is one call of one expert.
//
// Slots claim capacity in a priority order: token-major (ascending token, then slot) or
// slot-major (all first choices, then all second choices, ...; ascending token within a
// slot position).  The passes walk "virtual tokens" in that order: token-major, virtual
// token u is token u with its k slots; slot-major, u = j*T + t is the single slot (t, j).
// The kept slots of one expert are laid out in priority order (a stable counting sort).
//
// Three integer-only passes, bit-deterministic:
//   1. count:   per block of 256 virtual tokens, LDS histogram -> block_counts[b][e]
//   2. scan:    per expert, exclusive scan over blocks -> block_base[b][e]; counts,
//               kept = min(counts, C), offsets = exclusive scan of kept, n_dropped
//   3. scatter: rank of each slot inside its expert = block_base + earlier waves of
//               the block + earlier lanes of the wave; kept slots go to
//               perm[offsets[e] + rank], inv gets the row or -1
// A batch of at most 256 virtual tokens runs all three in one workgroup.
// Re-routing adds passes: the overflowed slots are listed in priority order (one
// workgroup), one wave walks them and gives each the best expert (by logit, lowest index
// on ties) outside the token's top-k and earlier re-routes that still has room (with at
// most 64 experts and 16384 tokens all its state is in registers and LDS; otherwise a
// general walk over the priority positions), then every slot's row is rebuilt, with the
// router-chosen rows of an expert first and its re-routed arrivals after them.
#include "moe_common.h"

#include <type_traits>

namespace moe {
namespace {

constexpr int DP_TOK = 256;   // virtual tokens per block (4 waves x 64 lanes, one per lane)

// Slot addressing in priority order (see above).
struct SlotMap {
  int64_t T;
  int k;
  bool slot_major;
  __device__ int64_t ntok() const { return slot_major ? T * k : T; }
  __device__ int kv() const { return slot_major ? 1 : k; }
  __device__ int64_t slot(int64_t u, int jv) const {
    return slot_major ? (u % T) * k + u / T : u * k + jv;
  }
};

__global__ __launch_bounds__(256) void dispatch_count_kernel(const int32_t* __restrict__ idx, SlotMap m, int E,
                                                             int32_t* __restrict__ block_counts) {
  __shared__ int32_t cnt[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += 256) cnt[e] = 0;
  __syncthreads();
  const int64_t u = static_cast<int64_t>(blockIdx.x) * DP_TOK + threadIdx.x;
  if (u < m.ntok())
    for (int j = 0; j < m.kv(); ++j) {
      const int32_t e = idx[m.slot(u, j)];
      if (static_cast<uint32_t>(e) < static_cast<uint32_t>(E)) atomicAdd(&cnt[e], 1);
    }
  __syncthreads();
  int32_t* out = block_counts + static_cast<int64_t>(blockIdx.x) * E;
  for (int e = threadIdx.x; e < E; e += 256) out[e] = cnt[e];
}

// Single workgroup of 1024 threads; thread e owns expert e.
__global__ __launch_bounds__(1024) void dispatch_scan_kernel(const int32_t* __restrict__ block_counts,
                                                             int nblocks, int E, int64_t capacity,
                                                             int32_t* __restrict__ block_base,
                                                             int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ n_dropped) {
  __shared__ int32_t wsum[16];
  __shared__ int32_t wdrop[16];
  const int e = threadIdx.x, lane = e & 63, wave = e >> 6;
  int32_t total = 0;
  if (e < E) {
    for (int b = 0; b < nblocks; ++b) {
      block_base[static_cast<int64_t>(b) * E + e] = total;
      total += block_counts[static_cast<int64_t>(b) * E + e];
    }
    counts[e] = total;
  }
  const int32_t kept = (e < E) ? (capacity > 0 && total > capacity ? static_cast<int32_t>(capacity) : total) : 0;
  int32_t drop = (e < E) ? total - kept : 0;
  // inclusive scan of kept across the workgroup (wave scan + wave totals)
  int32_t v = kept;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t o = __shfl_up(v, off);
    if (lane >= off) v += o;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) drop += __shfl_xor(drop, off);
  if (lane == 63) wsum[wave] = v;
  if (lane == 0) wdrop[wave] = drop;
  __syncthreads();
  int32_t before = 0, dsum = 0;
  for (int w = 0; w < 16; ++w) {
    if (w < wave) before += wsum[w];
    dsum += wdrop[w];
  }
  const int32_t incl = before + v;
  if (e < E) offsets[e + 1] = incl;
  if (e == 0) { offsets[0] = 0; *n_dropped = dsum; }
}

// Place the slots of one block of 256 tokens (one token per thread).  wcnt[w][e] must
// hold the per-wave demand of this block; block_base(e) is the number of earlier tokens
// (in earlier blocks) that chose e, offsets[e] the first row of e.
template <typename BaseFn>
__device__ void scatter_block(const int32_t* __restrict__ idx, SlotMap m, int E, int64_t capacity,
                              BaseFn block_base, const int32_t* offsets, int32_t (*wcnt)[kMaxExperts],
                              int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t u = static_cast<int64_t>(blockIdx.x) * DP_TOK + threadIdx.x;
  const bool valid = u < m.ntok();
  const int kv = m.kv();
  auto place = [&](int j, int32_t e, int32_t rank) {
    if (valid && e < 0) inv[m.slot(u, j)] = -1;
    if (e >= 0) {
      int32_t r = block_base(e) + rank;
      for (int w = 0; w < wave; ++w) r += wcnt[w][e];
      const int64_t slot = m.slot(u, j);
      if (capacity > 0 && r >= capacity) {
        inv[slot] = -1;
      } else {
        const int32_t row = offsets[e] + r;
        perm[row] = static_cast<int32_t>(slot);
        inv[slot] = row;
      }
    }
  };
  // rank of slot j inside its expert e among this wave's slots: the lanes below me
  // (earlier virtual tokens) that selected e in any of their slots, plus this token's
  // own earlier slots that selected e (a router never lists one expert twice, but a
  // caller's topk_idx may; the slots then take distinct rows in slot order, as the
  // token-major priority order (t, j) says).  Up to KMAX slots per virtual token, each lane's choices
  // stay in registers and every (slot, source lane) value is shuffled once for all of
  // this lane's slots: k*64 lane reads instead of k*k*64 (instantiated for 1, 2, 4 and 8
  // slots; more take the plain loop).  The source lane is a loop counter, the same in
  // every lane, so a scalar lane read does the job (every lane of the block is active).
  auto fast = [&](auto kmax) {
    constexpr int KMAX = decltype(kmax)::value;
    int32_t e[KMAX], raw[KMAX], rank[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      raw[j] = (j < kv && valid) ? idx[m.slot(u, j)] : -2;
      e[j] = (j < kv && static_cast<uint32_t>(raw[j]) < static_cast<uint32_t>(E)) ? raw[j] : -1;
      rank[j] = 0;
    }
#pragma unroll
    for (int j2 = 0; j2 < KMAX; ++j2) {
      if (j2 >= kv) break;
      for (int src = 0; src < 64; ++src) {
        const int32_t es = __builtin_amdgcn_readlane(raw[j2], src);   // uniform source lane
#pragma unroll
        for (int j = 0; j < KMAX; ++j) rank[j] += (src < lane && es == e[j]) ? 1 : 0;
      }
    }
#pragma unroll
    for (int j = 1; j < KMAX; ++j)
#pragma unroll
      for (int j2 = 0; j2 < j; ++j2) rank[j] += (e[j2] == e[j]) ? 1 : 0;
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (j < kv) place(j, e[j], rank[j]);
  };
  if (kv <= 1) return fast(std::integral_constant<int, 1>());
  if (kv <= 2) return fast(std::integral_constant<int, 2>());
  if (kv <= 4) return fast(std::integral_constant<int, 4>());
  if (kv <= 8) return fast(std::integral_constant<int, 8>());
  for (int j = 0; j < kv; ++j) {
    int32_t e = valid ? idx[m.slot(u, j)] : -1;
    if (static_cast<uint32_t>(e) >= static_cast<uint32_t>(E)) e = -1;   // ignored slot
    int32_t rank = 0;
    for (int j2 = 0; j2 < kv; ++j2) {
      const int32_t v = valid ? idx[m.slot(u, j2)] : -2;
      for (int src = 0; src < 64; ++src) {
        const int32_t es = __builtin_amdgcn_readlane(v, src);
        rank += (src < lane && es == e) ? 1 : 0;
      }
      rank += (j2 < j && e >= 0 && v == e) ? 1 : 0;     // this token's earlier slots
    }
    place(j, e, rank);
  }
}

// Per-wave demand of this block into wcnt (zeroed here).
__device__ void count_block(const int32_t* __restrict__ idx, SlotMap m, int E, int32_t (*wcnt)[kMaxExperts]) {
  const int wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 4 * E; i += 256) wcnt[i / E][i % E] = 0;
  __syncthreads();
  const int64_t u = static_cast<int64_t>(blockIdx.x) * DP_TOK + threadIdx.x;
  if (u < m.ntok())
    for (int j = 0; j < m.kv(); ++j) {
      const int32_t e = idx[m.slot(u, j)];
      if (static_cast<uint32_t>(e) < static_cast<uint32_t>(E)) atomicAdd(&wcnt[wave][e], 1);
    }
  __syncthreads();
}

__global__ __launch_bounds__(256) void dispatch_scatter_kernel(
    const int32_t* __restrict__ idx, SlotMap m, int E, int64_t capacity,
    const int32_t* __restrict__ block_base, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
  __shared__ int32_t wcnt[4][kMaxExperts];
  count_block(idx, m, E, wcnt);
  const int32_t* bb = block_base + static_cast<int64_t>(blockIdx.x) * E;
  scatter_block(idx, m, E, capacity, [&](int e) { return bb[e]; }, offsets, wcnt, perm, inv);
}

// All of dispatch in one workgroup when the batch fits one block (T <= 256): demand,
// kept counts, offsets and drops are computed in LDS, then the slots are placed.
__global__ __launch_bounds__(256) void dispatch_small_kernel(
    const int32_t* __restrict__ idx, SlotMap m, int E, int64_t capacity,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
    int32_t* __restrict__ inv, int32_t* __restrict__ n_dropped) {
  __shared__ int32_t wcnt[4][kMaxExperts];
  __shared__ int32_t off[kMaxExperts + 1];
  __shared__ int32_t wsum[4], wdrop[4];
  count_block(idx, m, E, wcnt);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // thread i owns experts 4i .. 4i+3 (E <= 1024)
  int32_t kept_loc[4];
  int32_t sum = 0, drop = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = threadIdx.x * 4 + q;
    int32_t c = 0, kept = 0;
    if (e < E) {
      c = wcnt[0][e] + wcnt[1][e] + wcnt[2][e] + wcnt[3][e];
      kept = (capacity > 0 && c > capacity) ? static_cast<int32_t>(capacity) : c;
      counts[e] = c;
    }
    kept_loc[q] = kept;
    sum += kept;
    drop += c - kept;
  }
  int32_t v = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t x = __shfl_up(v, o);
    if (lane >= o) v += x;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) drop += __shfl_xor(drop, o);
  if (lane == 63) wsum[wave] = v;
  if (lane == 0) wdrop[wave] = drop;
  __syncthreads();
  int32_t before = 0;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  int32_t run = before + v - sum;               // exclusive prefix of this thread's first expert
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = threadIdx.x * 4 + q;
    if (e < E) {
      off[e] = run;
      offsets[e] = run;
    }
    run += kept_loc[q];
  }
  if (threadIdx.x == 0) {
    const int32_t total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    off[E] = total;
    offsets[E] = total;
    *n_dropped = wdrop[0] + wdrop[1] + wdrop[2] + wdrop[3];
  }
  __syncthreads();
  scatter_block(idx, m, E, capacity, [](int) { return 0; }, off, wcnt, perm, inv);
}

// ---- re-routing of the overflow -------------------------------------------------
// Wave-wide maximum of a 64-bit key (hi, lo) with DPP lane moves (no LDS round trips):
// maxima inside 16-lane rows (quad_perm [1,0,3,2] = 0xB1, [2,3,0,1] = 0x4E, row_ror:4 =
// 0x124, row_ror:8 = 0x128), then across rows (row_bcast:15 = 0x142 into rows 1 and 3,
// row_bcast:31 = 0x143 into rows 2 and 3); lane 63 ends with the maximum, which is
// returned to every lane.
template <int CTRL, int ROWS>
__device__ __forceinline__ void key_max_dpp(uint32_t& hi, uint32_t& lo) {
  const uint32_t ohi = static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(static_cast<int>(hi), static_cast<int>(hi), CTRL, ROWS, 0xF, false));
  const uint32_t olo = static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(static_cast<int>(lo), static_cast<int>(lo), CTRL, ROWS, 0xF, false));
  if (ohi > hi || (ohi == hi && olo > lo)) { hi = ohi; lo = olo; }
}
__device__ __forceinline__ void wave_key_max(uint32_t& hi, uint32_t& lo) {
  key_max_dpp<0xB1, 0xF>(hi, lo);
  key_max_dpp<0x4E, 0xF>(hi, lo);
  key_max_dpp<0x124, 0xF>(hi, lo);
  key_max_dpp<0x128, 0xF>(hi, lo);
  key_max_dpp<0x142, 0xA>(hi, lo);
  key_max_dpp<0x143, 0xC>(hi, lo);
  hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(hi), 63));
  lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(lo), 63));
}

__device__ __forceinline__ uint32_t dp_ordered_key(float z) {
  uint32_t b = __float_as_uint(z);
  if (b == 0x80000000u) b = 0u;                       // -0 ties with +0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// One wave.  Walks the slots in priority order; a slot with a valid expert and no row
// (inv < 0 after the capacity pass) takes the best expert outside its token's top-k and
// the token's earlier re-routes that still has room.  Writes target[slot] (-1: still
// dropped), arrival[slot] (rank among the expert's re-routed arrivals), the new offsets
// (kept + arrivals; the capacity pass's offsets are saved to off1 first) and n_dropped.
// The walk goes in chunks of 64 priority positions; the logits and top-k rows of a
// chunk's overflowed slots are first staged into LDS together (one memory round trip
// per chunk, not per slot).  The experts a token already uses live in an LDS flag array:
// in token-major order a token's slots are consecutive, so the flags carry over between
// them; in slot-major order the targets of the token's earlier slot positions come from
// an LDS copy of `target` (when T*k fits) or are read back from memory past L1 after the
// stores that wrote them have completed.  One wave's LDS accesses execute in issue
// order, so flag and counter updates need only compiler ordering (signal fences).
struct RerouteLds {
  int chunk;         // priority positions per chunk (64, 32, 16 or 8)
  int stage_e;       // E (row length of the staged logits)
  int stage_k;       // k
  bool tcache;       // LDS copy of target[T*k] follows the staging area
};

// Dynamic LDS of the re-route pass: the staging rows of one chunk (at most 96 KB: the
// chunk shrinks for wide rows) and, in slot-major order, the target copy when it fits
// in the rest of 140 KB (the kernel's static arrays take another 16.5 KB of the 160 KB).
size_t reroute_lds_bytes(int64_t T, int E, int k, bool slot_major, RerouteLds& cfg) {
  const size_t row = static_cast<size_t>(E + k) * sizeof(int32_t);
  int chunk = 64;
  while (chunk > 8 && chunk * row > 96 * 1024) chunk /= 2;
  const size_t stage = chunk * row;
  const size_t tc = static_cast<size_t>(T) * k * sizeof(int32_t);
  cfg.chunk = chunk;
  cfg.stage_e = E;
  cfg.stage_k = k;
  cfg.tcache = stage + tc <= 140 * 1024;
  (void)slot_major;
  return stage + (cfg.tcache ? tc : 0);
}

__global__ __launch_bounds__(64) void dispatch_reroute_kernel(
    const int32_t* __restrict__ idx, const float* __restrict__ logits, SlotMap m, int E, int64_t capacity,
    RerouteLds lc, const int32_t* __restrict__ inv, int32_t* __restrict__ offsets, int32_t* __restrict__ off1,
    int32_t* __restrict__ target, int32_t* __restrict__ arrival, int32_t* __restrict__ n_dropped) {
  __shared__ int32_t room[kMaxExperts];
  __shared__ int32_t arr[kMaxExperts];
  __shared__ int32_t used[kMaxExperts];
  __shared__ int32_t kept1[kMaxExperts];
  __shared__ int64_t ctok[64];                       // token of each staged slot (-1: none)
  extern __shared__ __attribute__((aligned(16))) int32_t dyn[];
  float* zst = reinterpret_cast<float*>(dyn);        // [chunk][E] staged logits rows
  int32_t* kst = dyn + lc.chunk * lc.stage_e;        // [chunk][k] staged top-k rows
  int32_t* tcache = kst + lc.chunk * lc.stage_k;     // [T*k] when lc.tcache
  const int CH = lc.chunk;
  const int lane = threadIdx.x;
  const int k = m.k;
  const int64_t nslots = m.T * k;
  for (int e = lane; e <= E; e += 64) off1[e] = offsets[e];
  for (int e = lane; e < E; e += 64) {
    kept1[e] = offsets[e + 1] - offsets[e];
    room[e] = static_cast<int32_t>(capacity) - kept1[e];
    arr[e] = 0;
  }
  for (int64_t s = lane; s < nslots; s += 64) {
    target[s] = -1;
    if (lc.tcache) tcache[s] = -1;
  }
  const __amdgpu_buffer_rsrc_t trs =
      __builtin_amdgcn_make_buffer_rsrc(target, static_cast<short>(0), 0x7FFFFFFF, 0x00020000);
  __builtin_amdgcn_s_waitcnt(0);                      // target initialised before any read-back
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  const int32_t dropped1 = *n_dropped;
  int32_t moved = 0;
  int64_t cur_t = -1;
  // priority position p -> slot: token-major p itself, slot-major (p % T)*k + p / T;
  // lane i of a chunk holds position p0 + i (i < CH)
  for (int64_t p0 = 0; p0 < nslots; p0 += CH) {
    const int64_t p = p0 + lane;
    int32_t slot = -1, tok = -1, jj = 0;              // T*k < 2^29 for re-routing (host check)
    bool over = false;
    if (lane < CH && p < nslots) {
      slot = static_cast<int32_t>(m.slot_major ? (p % m.T) * k + p / m.T : p);
      tok = slot / k;
      jj = slot - tok * k;
      const int32_t e = idx[slot];
      over = static_cast<uint32_t>(e) < static_cast<uint32_t>(E) && inv[slot] < 0;
    }
    uint64_t mask = __ballot(over);
    if (!mask) continue;
    // stage the logits and top-k rows of this chunk's overflowed slots
    ctok[lane] = over ? tok : -1;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    for (int f = lane; f < CH * E; f += 64) {
      const int64_t t = ctok[f / E];
      if (t >= 0) zst[f] = logits[t * E + f % E];
    }
    for (int f = lane; f < CH * k; f += 64) {
      const int64_t t = ctok[f / k];
      if (t >= 0) kst[f] = idx[t * k + f % k];
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    // Decisions.  Fast path (target copy in LDS, E*k <= 8192): every pending slot picks
    // its best expert against the current room and its token's experts so far (top-k and
    // the targets of its earlier slots, final for slots of earlier chunks).  A pick still
    // open at the slot's turn is the greedy choice: room only shrinks and a token's
    // experts only grow, so the candidates at its turn are a subset of those it saw (and a
    // slot that saw none has none).  In priority order, a pick is still open if fewer
    // earlier picks of this run chose the same expert than it has room, and no earlier
    // slot of the same token in this run chose it.  The run up to the first pick that is
    // not open is applied at once (ranks counted across lanes); the rest pick again.
    // Slow path: one slot at a time with a wave-wide search.
    const bool fast = lc.tcache && E * k <= 8192;
    while (mask) {
      if (fast) {
        int32_t pick = -1;
        const bool mine = (mask >> lane) & 1;
        if (mine) {
          uint32_t bhi = 0, blo = 0;
          for (int e = 0; e < E; ++e) {
            if (room[e] <= 0) continue;
            bool excl = false;
            for (int q = 0; q < k; ++q) {
              excl |= kst[lane * k + q] == e;
              if (q < jj) excl |= tcache[tok * k + q] == e;
            }
            if (excl) continue;
            const uint32_t hi = dp_ordered_key(zst[lane * E + e]);
            const uint32_t lo = 0xffffffffu - static_cast<uint32_t>(e);
            if (hi > bhi || (hi == bhi && lo > blo)) { bhi = hi; blo = lo; }
          }
          pick = bhi != 0 ? static_cast<int32_t>(0xffffffffu - blo) : -1;
        }
        // rank among earlier picks of the same expert, and token clashes (readlane takes a
        // uniform lane index, so every lane walks all 64)
        int32_t before = 0;
        bool clash = false;
        for (int i2 = 0; i2 < 64; ++i2) {
          if (!((mask >> i2) & 1)) continue;          // uniform
          const int32_t pi = __builtin_amdgcn_readlane(pick, i2);
          const int32_t ti = __builtin_amdgcn_readlane(tok, i2);
          if (pi < 0 || pi != pick) continue;
          if (i2 < lane) {
            ++before;
            clash |= ti == tok;
          }
        }
        const bool closed = mine && pick >= 0 && (before >= room[pick] || clash);
        const uint64_t cmask = __ballot(closed);
        const uint64_t done = cmask ? (mask & ((uint64_t{1} << __builtin_ctzll(cmask)) - 1)) : mask;
        if (!done) {                                  // the first slot is not open: decide it alone
          goto one_slot;
        }
        {
          const bool take = ((done >> lane) & 1) && pick >= 0;
          // the last taker of an expert (no later taker in the run) updates its counters
          int32_t later = 0;
          for (int i2 = 0; i2 < 64; ++i2) {           // uniform lane index for readlane
            if (!((done >> i2) & 1)) continue;
            const int32_t pi = __builtin_amdgcn_readlane(pick, i2);
            later += (i2 > lane && pi == pick) ? 1 : 0;
          }
          int32_t a0 = 0, r0 = 0;
          if (take) {
            a0 = arr[pick];
            r0 = room[pick];
          }
          __atomic_signal_fence(__ATOMIC_SEQ_CST);
          if (take) {
            target[slot] = pick;
            arrival[slot] = a0 + before;
            tcache[slot] = pick;
            if (later == 0) {
              arr[pick] = a0 + before + 1;
              room[pick] = r0 - (before + 1);
            }
          }
          moved += static_cast<int32_t>(__builtin_popcountll(__ballot(take)));
          mask &= ~done;
          __atomic_signal_fence(__ATOMIC_SEQ_CST);
          continue;
        }
      }
    one_slot: {
        const int src = __builtin_ctzll(mask);
        const int32_t sl = __builtin_amdgcn_readlane(slot, src);
        const int64_t t = __builtin_amdgcn_readlane(tok, src);
        const int j = __builtin_amdgcn_readlane(jj, src);
        if (m.slot_major || t != cur_t || fast) {     // flags of the token: its top-k ...
          cur_t = t;
          for (int e = lane; e < E; e += 64) used[e] = 0;
          __atomic_signal_fence(__ATOMIC_SEQ_CST);
          for (int q = lane; q < k; q += 64) {
            const int32_t eq = kst[src * k + q];
            if (static_cast<uint32_t>(eq) < static_cast<uint32_t>(E)) used[eq] = 1;
            // ... and the targets of its earlier slots
            if (q < j && (m.slot_major || fast)) {
              const int32_t tg = lc.tcache ? tcache[t * k + q]
                                           : __builtin_amdgcn_raw_buffer_load_b32(
                                                 trs, static_cast<int>((t * k + q) * 4), 0, 1 /* glc: past L1 */);
              if (tg >= 0) used[tg] = 1;
            }
          }
          __atomic_signal_fence(__ATOMIC_SEQ_CST);
        }
        uint32_t bhi = 0, blo = 0;
        for (int ee = lane; ee < E; ee += 64) {
          if (room[ee] <= 0 || used[ee]) continue;
          const uint32_t hi = dp_ordered_key(zst[src * E + ee]);
          const uint32_t lo = 0xffffffffu - static_cast<uint32_t>(ee);
          if (hi > bhi || (hi == bhi && lo > blo)) { bhi = hi; blo = lo; }
        }
        wave_key_max(bhi, blo);
        const int32_t e = bhi != 0 ? static_cast<int32_t>(0xffffffffu - blo) : -1;
        mask &= mask - 1;
        if (e >= 0) {                                 // an expert with room
          const int32_t a = arr[e];
          __atomic_signal_fence(__ATOMIC_SEQ_CST);
          if (lane == 0) {
            room[e] = room[e] - 1;
            arr[e] = a + 1;
            used[e] = 1;
            if (lc.tcache) tcache[sl] = e;
            target[sl] = e;
            arrival[sl] = a;
          }
          ++moved;
          if (!lc.tcache) __builtin_amdgcn_s_waitcnt(0);   // before any read-back
          __atomic_signal_fence(__ATOMIC_SEQ_CST);
        }
      }
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);          // staging area reused by the next chunk
  }
  // new offsets: kept + arrivals, exclusive scan over experts (lane owns a range)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  const int per = (E + 63) / 64;
  int32_t local = 0;
  for (int i = 0; i < per; ++i) {
    const int e = lane * per + i;
    if (e < E) local += kept1[e] + arr[e];
  }
  int32_t incl = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t x = __shfl_up(incl, o);
    if (lane >= o) incl += x;
  }
  int32_t run = incl - local;
  for (int i = 0; i < per; ++i) {
    const int e = lane * per + i;
    if (e < E) {
      offsets[e] = run;
      run += kept1[e] + arr[e];
    }
  }
  if (lane == 63) offsets[E] = incl;
  if (lane == 0) *n_dropped = dropped1 - moved;
}

// ---- re-routing with at most 64 experts --------------------------------------------
// Overflow list: the slots that overflowed (a valid expert, no row after the capacity
// pass) in priority order, from one workgroup that walks the priority positions in
// blocks of 1024; every slot without a row gets target -1 here.
__global__ __launch_bounds__(1024) void reroute_list_kernel(const int32_t* __restrict__ idx,
                                                            const int32_t* __restrict__ inv, SlotMap m, int E,
                                                            int32_t* __restrict__ target,
                                                            int32_t* __restrict__ ovl, int32_t* __restrict__ n_over) {
  __shared__ int32_t wsum[16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t nslots = m.T * m.k;
  int32_t base = 0;
  for (int64_t p0 = 0; p0 < nslots; p0 += 1024) {
    const int64_t p = p0 + threadIdx.x;
    bool over = false;
    int32_t slot = 0;
    if (p < nslots) {
      slot = static_cast<int32_t>(m.slot_major ? (p % m.T) * m.k + p / m.T : p);
      if (inv[slot] < 0) {
        target[slot] = -1;
        over = static_cast<uint32_t>(idx[slot]) < static_cast<uint32_t>(E);
      }
    }
    const uint64_t b = __ballot(over);
    if (lane == 0) wsum[wave] = __builtin_popcountll(b);
    __syncthreads();
    int32_t before = base, total = base;
    for (int w = 0; w < 16; ++w) {
      before += w < wave ? wsum[w] : 0;
      total += wsum[w];
    }
    if (over) ovl[before + __builtin_popcountll(b & ((uint64_t{1} << lane) - 1))] = slot;
    base = total;
    __syncthreads();
  }
  if (threadIdx.x == 0) *n_over = base;
}

// One wave walks the overflow list in chunks of 64 entries (lane i holds entry c+i).  Expert
// e's room and re-routed arrivals live in lane e; each lane holds its token's logit row in
// registers and a mask of the experts the token may not take (its top-k, plus an LDS mask
// per token of the experts its earlier slots were re-routed to).  Every pending lane picks
// the best expert with room outside that mask (highest logit, lowest index on ties).  A
// pick is still the greedy choice at the lane's turn if fewer earlier lanes of the run
// picked the same expert than it has room and no earlier lane of the same token picked it
// (room only shrinks and a token's excluded set only grows), so the run up to the first
// pick that fails this is applied at once and the rest pick again; the first pending lane
// always succeeds, so every round makes progress.  Same-token entries are adjacent in
// token-major order: each re-picks (k-1 passes) with the picks of its token's earlier
// entries in the run added to its mask, which is the choice it would face after them, and
// a same-expert pick within k-1 lanes still ends the run; in slot-major order a run stops
// where the slot position changes, and within one slot position the tokens are distinct.
template <int EM>   // experts held per lane: E <= EM <= 64
__global__ __launch_bounds__(64) void reroute64_kernel(const int32_t* __restrict__ idx,
                                                       const float* __restrict__ logits, SlotMap m, int E,
                                                       int64_t capacity, const int32_t* __restrict__ ovl,
                                                       const int32_t* __restrict__ n_over_p,
                                                       int32_t* __restrict__ offsets, int32_t* __restrict__ off1,
                                                       int32_t* __restrict__ target, int32_t* __restrict__ arrival,
                                                       int32_t* __restrict__ n_dropped) {
  extern __shared__ uint64_t tused[];                   // [T]: experts the token's re-routes took
  const int lane = threadIdx.x;
  const int k = m.k;
  for (int64_t t = lane; t < m.T; t += 64) tused[t] = 0;
  int32_t kept = 0, room = 0, arr = 0;
  if (lane < E) {
    const int32_t o0 = offsets[lane], o1 = offsets[lane + 1];
    off1[lane] = o0;
    kept = o1 - o0;
    room = static_cast<int32_t>(capacity) - kept;
  }
  if (lane == 0) off1[E] = offsets[E];
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  const uint64_t emask = E >= 64 ? ~uint64_t{0} : (uint64_t{1} << E) - 1;
  const uint64_t below = (uint64_t{1} << lane) - 1;
  const int32_t n_over = *n_over_p;
  const int32_t dropped1 = *n_dropped;
  int32_t moved = 0;
  for (int32_t c0 = 0; c0 < n_over; c0 += 64) {
    const bool has = c0 + lane < n_over;
    const int32_t slot = has ? ovl[c0 + lane] : 0;
    const int32_t tok = slot / k, jj = slot - (slot / k) * k;
    float z[EM];
    uint64_t tk = 0;
#pragma unroll
    for (int e = 0; e < EM; ++e) z[e] = (has && e < E) ? logits[static_cast<int64_t>(tok) * E + e] : 0.f;
    for (int q = 0; q < k; ++q) {
      const int32_t eq = has ? idx[static_cast<int64_t>(tok) * k + q] : -1;
      if (static_cast<uint32_t>(eq) < static_cast<uint32_t>(E)) tk |= uint64_t{1} << eq;
    }
    uint64_t pending = __ballot(has);
    while (pending) {
      const uint64_t avail = __ballot(lane < E && room > 0) & emask;
      const bool mine = (pending >> lane) & 1;
      const uint64_t used = mine ? tused[tok] : 0;
      auto best_of = [&](uint64_t cand) {
        int32_t p = -1;
        float best = 0.f;
#pragma unroll
        for (int e = 0; e < EM; ++e) {
          if ((cand >> e) & 1) {
            if (p < 0 || z[e] > best) {
              best = z[e];
              p = e;
            }
          }
        }
        return p;
      };
      int32_t pick = mine ? best_of(avail & ~(tk | used)) : -1;
      if (!m.slot_major) {
        // a token's overflowed slots are adjacent: each slot also excludes the picks of
        // its token's earlier slots in this run (what it would see after them, if they
        // are taken in this run; if not, it is past the run's end anyway); k-1 passes
        // settle a chain of k slots
        for (int it = 1; it < k && it < 64; ++it) {
          uint64_t excl = 0;
          for (int d = 1; d < k && d < 64; ++d) {
            const int32_t tu = __shfl_up(tok, d), pu = __shfl_up(pick, d);
            if (lane >= d && ((pending >> (lane - d)) & 1) && tu == tok && pu >= 0) excl |= uint64_t{1} << pu;
          }
          if (mine) pick = best_of(avail & ~(tk | used | excl));
        }
      }
      // rank among earlier lanes of the run with the same pick, per distinct pick
      const int first = __builtin_ctzll(pending);
      int32_t before = 0;
      uint64_t rem = __ballot(mine && pick >= 0);
      while (rem) {
        const int32_t e = __builtin_amdgcn_readlane(pick, __builtin_ctzll(rem));
        const uint64_t me = __ballot(mine && pick == e);
        if (mine && pick == e) before = __builtin_popcountll(me & below);
        rem &= ~me;
      }
      bool clash = false;
      if (m.slot_major) {
        clash = jj != __builtin_amdgcn_readlane(jj, first);   // another slot position: next round
      } else {
        for (int d = 1; d < k && d < 64; ++d) {
          const int32_t tu = __shfl_up(tok, d), pu = __shfl_up(pick, d);
          clash |= lane >= d && ((pending >> (lane - d)) & 1) && tu == tok && pu == pick;
        }
      }
      const int32_t room_p = __shfl(room, pick < 0 ? 0 : pick);
      const bool closed = mine && pick >= 0 && (before >= room_p || clash);
      const uint64_t cmask = __ballot(closed);
      // (the first pending lane is never closed - its pick has room and nothing before it
      // in the run - so it is always done and every round makes progress)
      const uint64_t done = (cmask ? (pending & ((uint64_t{1} << __builtin_ctzll(cmask)) - 1)) : pending) |
                            (pending & (~pending + 1));
      const bool take = ((done >> lane) & 1) && pick >= 0;
      const int32_t arr_p = __shfl(arr, pick < 0 ? 0 : pick);
      if (take) {
        target[slot] = pick;
        arrival[slot] = arr_p + before;
        atomicOr(reinterpret_cast<unsigned long long*>(&tused[tok]), 1ull << pick);
      }
      // counters of the experts taken in this run
      uint64_t tm = __ballot(take);
      moved += __builtin_popcountll(tm);
      while (tm) {
        const int32_t e = __builtin_amdgcn_readlane(pick, __builtin_ctzll(tm));
        const uint64_t me = __ballot(take && pick == e);
        const int32_t n = __builtin_popcountll(me);
        if (lane == e) {
          room -= n;
          arr += n;
        }
        tm &= ~me;
      }
      pending &= ~done;
      // one wave's LDS accesses execute in issue order: the mask updates precede the next
      // round's reads once the compiler keeps them in order
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
    }
  }
  // new offsets: kept + arrivals, exclusive scan over experts (lane e holds expert e)
  int32_t incl = lane < E ? kept + arr : 0;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t x = __shfl_up(incl, o);
    if (lane >= o) incl += x;
  }
  if (lane < E) offsets[lane] = incl - (kept + arr);
  if (lane == E - 1) offsets[E] = incl;
  if (lane == 0) *n_dropped = dropped1 - moved;
}

// Rebuild rows after re-routing: a router-chosen kept slot keeps its rank inside its
// expert; a re-routed slot goes after its new expert's router-chosen rows.
__global__ __launch_bounds__(256) void dispatch_rebuild_kernel(
    const int32_t* __restrict__ idx, int64_t nslots, int E, const int32_t* __restrict__ off1,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ target,
    const int32_t* __restrict__ arrival, int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
  const int64_t s = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (s >= nslots) return;
  const int32_t r1 = inv[s];
  int32_t row = -1;
  if (r1 >= 0) {
    const int32_t e = idx[s];
    row = offsets[e] + (r1 - off1[e]);
  } else {
    const int32_t e = target[s];
    if (e >= 0) row = offsets[e] + (off1[e + 1] - off1[e]) + arrival[s];
  }
  inv[s] = row;
  if (row >= 0) perm[row] = static_cast<int32_t>(s);
}

}  // namespace

// Workspace for every policy: block tables sized for T*k virtual tokens, the saved
// offsets and the per-slot re-route target and arrival rank.
size_t dispatch_ws_bytes(int64_t T, int E, int k) {
  const int64_t nb = (T * k + DP_TOK - 1) / DP_TOK;
  return 2 * align_up(static_cast<size_t>(nb) * E * sizeof(int32_t), 256) +
         align_up(static_cast<size_t>(E + 1) * sizeof(int32_t), 256) +
         3 * align_up(static_cast<size_t>(T) * k * sizeof(int32_t), 256) + align_up(sizeof(int32_t), 256);
}

moe_status_t launch_dispatch(const int32_t* topk_idx, const float* logits, int64_t T, int E, int k,
                             int64_t capacity, int priority, int overflow, int32_t* counts, int32_t* offsets,
                             int32_t* perm, int32_t* inv, int32_t* n_dropped, void* ws, hipStream_t s) {
  const SlotMap m{T, k, priority == MOE_PRIORITY_SLOT};
  const int64_t ntok = m.slot_major ? T * k : T;
  const int64_t nb = (ntok + DP_TOK - 1) / DP_TOK;
  const int64_t nb_max = (T * k + DP_TOK - 1) / DP_TOK;
  WsCarver c(ws);
  int32_t* block_counts = c.take<int32_t>(static_cast<size_t>(nb_max) * E);
  int32_t* block_base = c.take<int32_t>(static_cast<size_t>(nb_max) * E);
  int32_t* off1 = c.take<int32_t>(static_cast<size_t>(E) + 1);
  int32_t* target = c.take<int32_t>(static_cast<size_t>(T) * k);
  int32_t* arrival = c.take<int32_t>(static_cast<size_t>(T) * k);
  int32_t* ovl = c.take<int32_t>(static_cast<size_t>(T) * k);
  int32_t* n_over = c.take<int32_t>(1);
  if (nb <= 1) {
    const SlotMap mg{nb == 0 ? 0 : T, k, m.slot_major};
    dispatch_small_kernel<<<1, 256, 0, s>>>(topk_idx, mg, E, capacity, counts, offsets, perm, inv, n_dropped);
    if (moe_status_t st = check_launch("dispatch kernel")) return st;
  } else {
    dispatch_count_kernel<<<static_cast<unsigned>(nb), 256, 0, s>>>(topk_idx, m, E, block_counts);
    if (moe_status_t st = check_launch("dispatch count kernel")) return st;
    dispatch_scan_kernel<<<1, 1024, 0, s>>>(block_counts, static_cast<int>(nb), E, capacity, block_base,
                                            counts, offsets, n_dropped);
    if (moe_status_t st = check_launch("dispatch scan kernel")) return st;
    dispatch_scatter_kernel<<<static_cast<unsigned>(nb), 256, 0, s>>>(topk_idx, m, E, capacity,
                                                                      block_base, offsets, perm, inv);
    if (moe_status_t st = check_launch("dispatch scatter kernel")) return st;
  }
  if (overflow != MOE_OVERFLOW_REROUTE || capacity <= 0 || T == 0) return MOE_OK;
  const int64_t nslots = T * k;
  if (E <= 64 && T <= 16384) {
    reroute_list_kernel<<<1, 1024, 0, s>>>(topk_idx, inv, m, E, target, ovl, n_over);
    if (moe_status_t st = check_launch("dispatch overflow-list kernel")) return st;
    const size_t lds = static_cast<size_t>(T) * sizeof(uint64_t);
    auto run = [&](auto kern) {
      set_max_dynamic_smem(reinterpret_cast<const void*>(kern), lds);
      kern<<<1, 64, lds, s>>>(topk_idx, logits, m, E, capacity, ovl, n_over, offsets, off1, target, arrival,
                              n_dropped);
    };
    // the per-round argmax and the logit row cover EM experts per lane
    if (E <= 16) run(reroute64_kernel<16>);
    else if (E <= 32) run(reroute64_kernel<32>);
    else run(reroute64_kernel<64>);
    if (moe_status_t st = check_launch("dispatch re-route kernel")) return st;
    dispatch_rebuild_kernel<<<static_cast<unsigned>((nslots + 255) / 256), 256, 0, s>>>(
        topk_idx, nslots, E, off1, offsets, target, arrival, perm, inv);
    return check_launch("dispatch rebuild kernel");
  }
  RerouteLds lc{};
  const size_t lds = reroute_lds_bytes(T, E, k, m.slot_major, lc);
  set_max_dynamic_smem(reinterpret_cast<const void*>(dispatch_reroute_kernel), lds);
  dispatch_reroute_kernel<<<1, 64, lds, s>>>(topk_idx, logits, m, E, capacity, lc, inv, offsets, off1, target,
                                             arrival, n_dropped);
  if (moe_status_t st = check_launch("dispatch re-route kernel")) return st;
  dispatch_rebuild_kernel<<<static_cast<unsigned>((nslots + 255) / 256), 256, 0, s>>>(
      topk_idx, nslots, E, off1, offsets, target, arrival, perm, inv);
  return check_launch("dispatch rebuild kernel");
}

}  // namespace moe
