// Grouped expert FFN.  [cnnet] "MoE混合专家架构原理与工程实践…": expert weights stacked in
// one tensor and sliced by index, the tokens of one expert computed together;
// [200B-5] "四个专家同时算…": the vectors bound for one expert are batched.
//
// Each group (expert) owns a contiguous range of rows of the expert-sorted order.
// Two grouped GEMMs, both C[m, n] = sum_k A[m, k] B[n, k] with K-contiguous operands:
//   up:   A = x rows gathered through the permutation, B = W_gate (and W_up) [F, d];
//         epilogue silu(g) * u (SwiGLU) or gelu(g), rounded once to bf16 -> H [rows, F]
//   down: A = H rows, B = W_down [d, F] -> y [rows, d] fp32 (optionally split over K)
// A device-side schedule (one tiny kernel) turns the group offsets into M-tiles, so
// no host synchronisation is needed to learn how many rows each expert received.
//
// bf16 tile: up to 256 rows x 256 MFMA columns x 64 K per stage, 8 waves (2 per SIMD)
// (tile heights 32, 64, 128, 192 and 256 rows).
// Wave w owns 32 columns of every row of the tile: its weight fragments are private to
// it and are loaded straight from global memory into registers in the MFMA operand
// layout (no LDS; in the packed weight layout each such load reads one contiguous KiB),
// while the activation tile is shared by the 8 waves through a ring of 3 LDS slots,
// written by buffer-to-LDS loads (no register round trip), 16-byte chunks XOR-swizzled
// by row.  Only the 16-row fragments that hold real rows are multiplied,
// so a group with 70 rows costs 5 fragments, not 16.  Workgroups are remapped so that
// each XCD (blockIdx % 8) walks a contiguous range of tiles: the tiles of one expert
// share its activation rows in that XCD's L2.
#include "moe_common.h"
#include <type_traits>

namespace moe {
namespace {

constexpr int BM = 256;          // rows per M-tile (bf16)
constexpr int BK = 64;           // K per pipeline stage
constexpr int BM_F32 = 64;       // rows per M-tile (fp32 path)
constexpr int WEIGHT_RING = 3;   // weight register slots per wave (2 stages in flight)
constexpr int ACT_DIST = 2;      // stages the buffer-to-LDS activation loads run ahead

constexpr int gcd_c(int a, int b) { return b == 0 ? a : gcd_c(b, a % b); }

enum GemmMode { MODE_SWIGLU_UP = 0, MODE_GELU_UP = 1, MODE_DOWN = 2 };

// Schedule layout (int32 words in the workspace):
//   [0] total M-tiles, [1 .. Gt+1] exclusive prefix of M-tiles per group,
//   then row0[Gt], rows[Gt].
struct SchedView {
  const int32_t* base;
  int Gt;
  __device__ int32_t total() const { return base[0]; }
  __device__ const int32_t* prefix() const { return base + 1; }
  __device__ const int32_t* row0() const { return base + 2 + Gt; }
  __device__ const int32_t* rows() const { return base + 2 + 2 * Gt; }
  __device__ const int32_t* m2g() const { return base + 2 + 3 * Gt; }   // M-tile -> its group
};

// [total M-tiles][prefix: Gt + 1][row0: Gt][rows: Gt][group of each M-tile: max_mtiles]
inline size_t sched_words(int Gt, int64_t max_mtiles) {
  return 2 + 3 * static_cast<size_t>(Gt) + static_cast<size_t>(max_mtiles);
}

__global__ __launch_bounds__(1024) void ffn_schedule_kernel(const int32_t* __restrict__ offsets, int G,
                                                            int64_t max_rows, int64_t shared_rows,
                                                            int64_t shared_row0, int bm, int64_t max_mtiles,
                                                            int32_t* __restrict__ sched) {
  __shared__ int32_t wsum[16];
  const int Gt = G + (shared_rows > 0 ? 1 : 0);
  int32_t* prefix = sched + 1;
  int32_t* row0 = sched + 2 + Gt;
  int32_t* rows = sched + 2 + 2 * Gt;
  int32_t carry = 0;
  for (int g0 = 0; g0 < Gt; g0 += 1024) {
    const int g = g0 + threadIdx.x;
    int32_t mt = 0;
    if (g < Gt) {
      int64_t r0, r1;
      if (g < G) {
        r0 = offsets[g];
        r1 = offsets[g + 1];
        r0 = r0 < 0 ? 0 : (r0 > max_rows ? max_rows : r0);
        r1 = r1 < r0 ? r0 : (r1 > max_rows ? max_rows : r1);
      } else {
        r0 = shared_row0;
        r1 = shared_row0 + shared_rows;
      }
      row0[g] = static_cast<int32_t>(r0);
      rows[g] = static_cast<int32_t>(r1 - r0);
      mt = static_cast<int32_t>((r1 - r0 + bm - 1) / bm);
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int32_t v = mt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int32_t o = __shfl_up(v, off);
      if (lane >= off) v += o;
    }
    if (lane == 63) wsum[wave] = v;
    __syncthreads();
    int32_t before = carry, all = carry;
    for (int w = 0; w < 16; ++w) {
      if (w < wave) before += wsum[w];
      all += wsum[w];
    }
    if (g < Gt) prefix[g] = before + v - mt;
    carry = all;
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    prefix[Gt] = carry;
    sched[0] = carry;
  }
  // the group of every M-tile, so a workgroup finds its group with one load (the prefix
  // entries of other threads are visible after the loop's last barrier)
  int32_t* m2g = sched + 2 + 3 * Gt;
  for (int g = threadIdx.x; g < Gt; g += 1024) {
    const int32_t end = g + 1 < Gt ? prefix[g + 1] : carry;
    for (int32_t m = prefix[g]; m < end && m < max_mtiles; ++m) m2g[m] = g;
  }
}

struct GemmArgs {
  const uint16_t* a;        // x [n_x, K] (up) or H [rows, K] (down); fp32 data for the fp32 path
  const int32_t* perm;      // up only: nullable
  int k_div;                // perm entries divided by this give the token
  const void* w0;           // gate / W1 / Wd, stacked [G, N_w, K]
  const void* w1;           // up (SwiGLU) or null
  const void* sw0;          // shared-group weights
  const void* sw1;
  const int32_t* sched;
  int64_t max_mtiles;       // bound of the M-tile count (size of the schedule's group table)
  int G, Gt;
  int64_t shared_row0;
  int64_t K, N;             // contraction and output width (F for up, d for down)
  int nt;                   // N-tiles per M-tile
  int splits;               // K splits (down only)
  int64_t k_chunk;          // K per split (multiple of BK)
  void* out;                // H (bf16 or f32) or y / partials (f32)
  int64_t split_stride;     // elements between split partial buffers
};

// Locate the logical tile: group, M-tile, N-tile, split.
struct TileInfo {
  int g;
  int64_t row_begin;
  int nrows;
  int ntile;
  int split;
};

__device__ __forceinline__ bool decode_tile(const GemmArgs& p, int bm, TileInfo& ti) {
  const SchedView sv{p.sched, p.Gt};
  const int64_t nts = static_cast<int64_t>(p.nt) * p.splits;
  // (offsets that break their contract could claim more M-tiles than the table holds)
  const int64_t mtiles = sv.total() < p.max_mtiles ? sv.total() : p.max_mtiles;
  const int64_t n_active = mtiles * nts;
  const int64_t per_xcd = (n_active + 7) / 8;
  const int64_t b = blockIdx.x;
  const int64_t slot = b >> 3;
  if (slot >= per_xcd) return false;
  const int64_t L = (b & 7) * per_xcd + slot;
  if (L >= n_active) return false;
  // group g holds tiles [prefix[g] * nts, prefix[g+1] * nts), i.e. M-tiles prefix[g] ..
  // prefix[g+1]-1 in group order: its group is one table load away
  const int32_t* pre = sv.prefix();
  const int g = sv.m2g()[L / nts];
  // Inside a group the tiles go in blocks of up to MB M-tiles: all N-tiles (and K splits)
  // of one block, M fastest, then the next block.  The workgroups running at once on an
  // XCD then share both the weights of a few N-tiles and the activation rows of a few
  // M-tiles in its L2 (with M fastest over a whole large group, every round of N-tiles
  // would re-read all of the group's activation rows).
  const int64_t local = L - static_cast<int64_t>(pre[g]) * nts;
  const int mt = pre[g + 1] - pre[g];
  constexpr int MB = 4;
  const int A = mt < MB ? mt : MB;
  const int nfull = mt / A;
  const int64_t in_full = static_cast<int64_t>(nfull) * A * nts;
  int64_t j;
  int m;
  if (local < in_full) {
    const int64_t mb = local / (static_cast<int64_t>(A) * nts);
    const int64_t r = local - mb * A * nts;
    j = r / A;
    m = static_cast<int>(mb * A + (r - j * A));
  } else {                                    // the last, partial block
    const int A2 = mt - nfull * A;
    const int64_t r = local - in_full;
    j = r / A2;
    m = nfull * A + static_cast<int>(r - j * A2);
  }
  ti.g = g;
  ti.ntile = static_cast<int>(j / p.splits);
  ti.split = static_cast<int>(j - static_cast<int64_t>(ti.ntile) * p.splits);
  ti.row_begin = static_cast<int64_t>(sv.row0()[g]) + static_cast<int64_t>(m) * bm;
  const int rem = sv.rows()[g] - m * bm;
  ti.nrows = rem < bm ? rem : bm;
  return true;
}

// Raw buffer resource over [base, base + 2^31): every offset the GEMM forms is below 2^31
// (x and one expert's weights are below 2 GiB, checked on the host; H is addressed from
// each tile's first row), so the range check only ever refuses deliberate out-of-range
// offsets.
constexpr uint32_t OOB_OFFSET = 0x80000000u;   // beyond the 2^31 - 1 byte buffer range

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), 0x7FFFFFFF, 0x00020000);
}

// ---- epilogue stores.  In the MFMA C layout a lane holds rows 4 (lane / 16) + v, v = 0..3,
// of one column (lane % 16) of a 16 x 16 block, so a plain store writes 2 or 4 bytes per
// lane.  The 4 lanes of a quad hold 4 adjacent columns of the same 4 rows: a 4 x 4
// transpose inside the quad (two DPP swaps, at distance 2 then 1) leaves lane t of the quad
// with row t, columns 0..3, so each lane writes one 8-byte (bf16) or 16-byte (fp32) store.
// Every lane of the quad must be active.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t quad_swap2(uint32_t v) {   // lanes t <-> t ^ 2
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x4E, 0xF, 0xF, false));
}
__device__ __forceinline__ uint32_t quad_swap1(uint32_t v) {   // lanes t <-> t ^ 1
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// h[v] = rows v of this lane's column -> the 4 bf16 of row (lane % 4), columns 0..3 of the quad.
__device__ __forceinline__ u32x2 quad_rows_bf16(const float h[4], int lane) {
  const int t = lane & 3;
  const uint32_t a = pack_bf16(h[0], h[1]), b = pack_bf16(h[2], h[3]);
  const bool low = t < 2, odd = t & 1;
  const uint32_t recv = quad_swap2(low ? b : a);
  const uint32_t X = low ? a : recv;            // column t % 2 of rows r0, r0 + 1 (r0 = t & 2)
  const uint32_t Y = low ? recv : b;            // column t % 2 + 2 of the same rows
  // odd lanes hand over row r0 (low halves), even lanes row r0 + 1 (high halves)
  const uint32_t r2 = quad_swap1(__builtin_amdgcn_perm(Y, X, odd ? 0x05040100u : 0x07060302u));
  u32x2 o;
  o.x = odd ? __builtin_amdgcn_perm(X, r2, 0x07060100u) : __builtin_amdgcn_perm(r2, X, 0x05040100u);
  o.y = odd ? __builtin_amdgcn_perm(Y, r2, 0x07060302u) : __builtin_amdgcn_perm(r2, Y, 0x07060100u);
  return o;
}

// The same for fp32 values: the 4 floats of row (lane % 4), columns 0..3 of the quad.
__device__ __forceinline__ f32x4 quad_rows_f32(const f32x4& v, int lane) {
  const int t = lane & 3;
  const bool low = t < 2, odd = t & 1;
  const float q0 = __uint_as_float(quad_swap2(__float_as_uint(low ? v[2] : v[0])));
  const float q1 = __uint_as_float(quad_swap2(__float_as_uint(low ? v[3] : v[1])));
  const float X0 = low ? v[0] : q0, X1 = low ? v[1] : q1;   // column t % 2
  const float Y0 = low ? q0 : v[2], Y1 = low ? q1 : v[3];   // column t % 2 + 2
  const float w0 = __uint_as_float(quad_swap1(__float_as_uint(odd ? X0 : X1)));
  const float w1 = __uint_as_float(quad_swap1(__float_as_uint(odd ? Y0 : Y1)));
  return odd ? f32x4{w0, X1, w1, Y1} : f32x4{X0, w0, Y0, w1};
}

// First row of the A operand's buffer resource: the tile's first row for the down
// projection (A = H, read row by row), row 0 for the up projection (A = x, rows gathered).
__device__ __forceinline__ int64_t a_base_row(int mode, const TileInfo& ti) {
  return mode == MODE_DOWN ? ti.row_begin : 0;
}

// Source row of the A operand for output row r of group g.
__device__ __forceinline__ int64_t a_source_row(const GemmArgs& p, int mode, int g, int64_t r) {
  if (mode == MODE_DOWN) return r;
  if (g >= p.G) return r - p.shared_row0;           // shared group: identity rows
  return p.perm ? static_cast<int64_t>(p.perm[r] / p.k_div) : r;
}

// Tile: MT*16 rows x 256 MFMA columns, K advanced BK=64 per pipeline stage, NW waves of
// NF 16-column fragments each (NW * NF * 16 = 256).  With NW = 8 two waves share each
// SIMD, so one wave's memory and LDS latency hides behind the other's MFMAs.
// Weights: a ring of WRING register slots per wave (stage s is multiplied while the next
// WRING-1 stages are in flight).  Activations: buffer-to-LDS loads D stages ahead into a
// ring of D+1 LDS slots (when the tile has at least one 16-byte chunk per thread; smaller
// tiles go through a 2-slot register ring and LDS stores, two stages ahead).  Every global load
// is issued unconditionally (padding rows take an out-of-range offset, which returns zeros
// without touching memory, and inactive waves read valid weight rows; neither result is
// stored) so the memory counters stay in step across waves, and activation loads are
// issued before weight loads so that waiting
// for one stage's activations never waits for weights.  Loads are raw buffer loads:
// uniform base, 32-bit per-lane offset, uniform stage offset.  The LDS slots arrive as
// distinct restrict pointers so the compiler can tell a slot being read from the slots
// being filled and does not wait for those loads before its LDS reads.
template <int MODE, int MT, int NW, bool PK>
__device__ __forceinline__ void ffn_gemm_bf16_body(const GemmArgs& p, uint16_t* __restrict__ L0,
                                                   uint16_t* __restrict__ L1, uint16_t* __restrict__ L2,
                                                   uint16_t* __restrict__ L3) {
  constexpr int NT = NW * 64;                     // threads
  constexpr int NF = 256 / (16 * NW);             // 16-column fragments per wave
  constexpr int WCOLS = NF * 16;                  // MFMA columns per wave
  constexpr int BMT = MT * 16;
  constexpr int AR = (BMT * 8 + NT - 1) / NT;     // 16-byte activation chunks per thread per stage
  constexpr bool WRAP = (AR * NT / 8) > BMT;      // fewer chunks than threads: register path
  constexpr int D = WRAP ? 2 : ACT_DIST;          // activation prefetch distance (stages)
  constexpr int LRING = D + 1;                    // LDS activation slots
  constexpr int WRING = WEIGHT_RING;
  static_assert(D <= WRING - 1 && LRING <= 4, "weights run at least as far ahead as activations");
  // With one fragment per wave (16 waves), a SwiGLU wave's 16 columns pair 8 gate rows
  // (lanes with lane%16 < 8) with the 8 up rows of the same hidden units (lane%16 >= 8).
  constexpr bool PAIRED = MODE == MODE_SWIGLU_UP && NF == 1;
  static_assert(NF >= 1 && NF * 16 * NW == 256, "tile shape");
  auto lds = [&](int slot) -> uint16_t* { return slot == 0 ? L0 : slot == 1 ? L1 : slot == 2 ? L2 : L3; };
  TileInfo ti;
  if (!decode_tile(p, BMT, ti)) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nmf = (ti.nrows + 15) >> 4;

  // ---- K range of this tile
  int64_t k_begin = 0, k_end = p.K;
  if (MODE == MODE_DOWN && p.splits > 1) {
    k_begin = static_cast<int64_t>(ti.split) * p.k_chunk;
    k_end = k_begin + p.k_chunk < p.K ? k_begin + p.k_chunk : p.K;
  }
  const int nst = k_end > k_begin ? static_cast<int>((k_end - k_begin) / BK) : 0;

  // ---- weight rows (columns of C) owned by this wave.  SwiGLU: the first half of the
  // fragments are gate rows, the second half the up rows of the same hidden units.
  const bool shared_grp = ti.g >= p.G;
  const int64_t wstride = shared_grp ? 0 : static_cast<int64_t>(ti.g) * p.N * p.K;
  const char* Wb0 = reinterpret_cast<const char*>(static_cast<const uint16_t*>(shared_grp ? p.sw0 : p.w0) + wstride);
  const char* Wb1 = reinterpret_cast<const char*>(static_cast<const uint16_t*>(shared_grp ? p.sw1 : p.w1) + wstride);
  if (MODE != MODE_SWIGLU_UP) Wb1 = Wb0;
  // Weight byte offsets.  Linear layout [N_w, K]: lane (row, kgroup) reads 8 elements at
  // K = 8*kgroup of its row; the two k32 steps of a stage are 64 B apart, stages 128 B,
  // and one load covers 64 contiguous bytes of each of 16 rows.  Packed layout
  // [N_w/16][K/32][64 lanes][8]: each 16-row x 32-K fragment is one contiguous KiB in
  // lane order, so one load reads 1 KiB contiguous; k32 steps 1 KiB apart, stages 2 KiB.
  constexpr int W_STEP = PK ? 1024 : 64;
  constexpr int W_STAGE = PK ? 2048 : BK * 2;
  auto woff = [&](int64_t row) -> uint32_t {
    const int kg = lane >> 4;
    if (PK) return static_cast<uint32_t>((((row >> 4) * (p.K >> 5) + (k_begin >> 5)) * 64 + (row & 15) + 16 * kg) * 16);
    return static_cast<uint32_t>((row * p.K + k_begin + 8 * kg) * 2);
  };
  int64_t col_base;                         // first output column of this wave
  if (MODE == MODE_SWIGLU_UP) col_base = static_cast<int64_t>(ti.ntile) * 128 + wave * (WCOLS / 2);   // hidden unit
  else col_base = static_cast<int64_t>(ti.ntile) * 256 + wave * WCOLS;
  const bool wave_on = col_base < p.N;
  uint32_t boff[NF];                        // byte offsets of this lane's weight rows
#pragma unroll
  for (int nf = 0; nf < NF; ++nf) {
    int64_t wrow = PAIRED ? col_base + (lane & 7)
                 : (MODE == MODE_SWIGLU_UP) ? col_base + (nf % (NF / 2)) * 16 + (lane & 15)
                                            : col_base + nf * 16 + (lane & 15);
    if (!wave_on) wrow = lane & 15;         // a valid row; the result is not stored
    boff[nf] = woff(wrow);
  }
  // paired layout: this lane's weight row lives in the gate or the up tensor
  const char* wlane = PAIRED ? ((lane & 8) ? Wb1 : Wb0) + boff[0] : nullptr;

  // ---- activation chunks loaded by this thread: chunk q = i*NT + tid -> row q/8 (mod
  // the tile height; a repeated row writes identical bytes), 16-byte column q%8 = tid%8.
  // The XOR swizzle uses row%8 = (tid/8)%8 for every i (NT/8 is a multiple of 8).
  // H (the down projection's A) is addressed from the tile's first row, so its offsets stay
  // below 2^31 however many rows H has; x is addressed from its start (gathered rows).
  const int64_t a_row0 = a_base_row(MODE, ti);
  const char* Ab = reinterpret_cast<const char*>(p.a) + a_row0 * p.K * 2;
  const int chunk = tid & 7;
  uint32_t aoff[AR];
#pragma unroll
  for (int i = 0; i < AR; ++i) {
    const int r = WRAP ? ((i * NT + tid) >> 3) % BMT : (i * NT + tid) >> 3;
    // padding rows get an offset past the buffer's range: the load returns zeros without
    // touching memory (their rows are never stored), and still counts for the waits
    const int cc = WRAP ? chunk : (chunk ^ (r & 7));
    aoff[i] = r < ti.nrows ? static_cast<uint32_t>(((a_source_row(p, MODE, ti.g, ti.row_begin + r) - a_row0) * p.K +
                                                    k_begin + cc * 8) * 2)
                           : OOB_OFFSET;
  }
  // Buffer resources: uniform base + 32-bit per-lane offset + uniform stage offset.
  const __amdgpu_buffer_rsrc_t arsrc = make_rsrc(Ab);
  const __amdgpu_buffer_rsrc_t w0rsrc = make_rsrc(Wb0);
  const __amdgpu_buffer_rsrc_t w1rsrc = make_rsrc(Wb1);
  const int st_row0 = WRAP ? (tid >> 3) % BMT : (tid >> 3);
  const int st_off0 = st_row0 * BK + ((chunk ^ (st_row0 & 7)) * 8);   // element offset in a slot

  u32x4 ra[2][AR];                          // activation register ring: 2 stages
  bf16x8 rb[WRING][2][NF];                  // weight register ring: [slot][k32 step][fragment]

  auto clamp_stage = [&](int st) { return st < 0 ? 0 : (st < nst ? st : nst - 1); };
  auto load_a = [&](int st, int aslot, int lslot) {
    st = clamp_stage(st);
    const int ko = st * (BK * 2);           // uniform part of the offset
    if (WRAP) {
#pragma unroll
      for (int i = 0; i < AR; ++i) ra[aslot][i] = __builtin_amdgcn_raw_buffer_load_b128(arsrc, aoff[i], ko, 0);
    } else {
#pragma unroll
      for (int i = 0; i < AR; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(arsrc,
            (__attribute__((address_space(3))) void*)(lds(lslot) + (i * (NT / 64) + wave) * 512), 16, aoff[i], ko, 0, 0);
    }
  };
  // Make the activations of a stage visible: with buffer-to-LDS loads, wait until this
  // wave's loads of that stage have landed (the loads issued after them: 2 stages of
  // weights, 2*NF each, and one stage of activations, AR) - the barrier that follows
  // makes every wave's share visible.  Otherwise store the register copy into LDS.
  auto store_a = [&](int aslot, int lslot) {
    if (!WRAP) {
      constexpr int N = D * 2 * NF + (D - 1) * AR;
      static_assert(N < 64, "vmcnt range");
      // s_waitcnt immediate (gfx9 layout): vmcnt in [3:0] and [15:14], expcnt [6:4] and
      // lgkmcnt [11:8] left at their maxima (no wait)
      __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
      return;
    }
#pragma unroll
    for (int i = 0; i < AR; ++i) {
      if (WRAP) {
        const int r = ((i * NT + tid) >> 3) % BMT;
        *reinterpret_cast<u32x4*>(&lds(lslot)[r * BK + ((chunk ^ (r & 7)) * 8)]) = ra[aslot][i];
      } else {
        *reinterpret_cast<u32x4*>(&lds(lslot)[st_off0 + i * (NT / 8) * BK]) = ra[aslot][i];
      }
    }
  };
  auto load_b = [&](int st, int slot) {
    st = clamp_stage(st);
    const int ko = st * W_STAGE;            // uniform part of the offset
    if (PAIRED) {                           // per-lane tensor: a 64-bit address
#pragma unroll
      for (int s = 0; s < 2; ++s) rb[slot][s][0] = *reinterpret_cast<const bf16x8*>(wlane + ko + s * W_STEP);
      return;
    }
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int nf = 0; nf < NF; ++nf) {
        const auto& rs = (MODE == MODE_SWIGLU_UP && nf >= NF / 2) ? w1rsrc : w0rsrc;
        rb[slot][s][nf] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rs, boff[nf] + s * W_STEP, ko, 0));
      }
  };
  // One load of a phase by index, in the phase's issue order: the AR activation chunks of
  // stage sta, then the 2*NF weight fragments of stage stb (k32 step major).
  auto load_one = [&](int idx, int sta, int lslot, int stb, int bslot) {
    if (idx < AR) {
      const int ko = clamp_stage(sta) * (BK * 2);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(arsrc,
          (__attribute__((address_space(3))) void*)(lds(lslot) + (idx * (NT / 64) + wave) * 512), 16, aoff[idx], ko,
          0, 0);
    } else {
      const int w = idx - AR, s = w / NF, nf = w % NF;
      const int ko = clamp_stage(stb) * W_STAGE;
      if (PAIRED) {
        rb[bslot][s][0] = *reinterpret_cast<const bf16x8*>(wlane + ko + s * W_STEP);
      } else {
        const auto& rs = (MODE == MODE_SWIGLU_UP && nf >= NF / 2) ? w1rsrc : w0rsrc;
        rb[bslot][s][nf] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rs, boff[nf] + s * W_STEP, ko, 0));
      }
    }
  };
  // Mark a weight slot as consumed on every path (the MFMAs that read it sit behind the
  // row-count guards), so its registers can be reloaded without a memory wait.
  auto consume_b = [&](int slot) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int nf = 0; nf < NF; ++nf) asm volatile("" ::"v"(rb[slot][s][nf]));
  };
  auto read_a = [&](int slot, int s, int mf) {
    const int r = mf * 16 + (lane & 15);
    const int c = (s * 4 + (lane >> 4)) ^ (r & 7);
    return *reinterpret_cast<const bf16x8*>(&lds(slot)[r * BK + c * 8]);
  };

  f32x4 acc[MT][NF];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NF; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Multiply one stage.  Activation fragments are read from LDS in groups of GS so one
  // LDS latency covers GS*NF MFMAs; groups past the tile's last real row are skipped.
  // The next group is read before the current group's MFMAs, so the LDS latency hides
  // behind them (measured: 5% on the MFMA-bound shared+routed layer, 2.5% on prefill);
  // 16 waves of 256 rows have no registers to spare for that.
  constexpr int GS = MT < 4 ? MT : 4;
  constexpr int NG = 2 * (MT / GS);          // groups per stage: 2 k32 steps x MT/GS
  constexpr bool PREFETCH = MT <= 8 || NW <= 8;
  // With spread loads, the activation chunks of the next stage go first, in one burst,
  // and group q then issues weight fragments [q*NW2/NG, (q+1)*NW2/NG) (every path issues
  // them all), so the memory pipeline takes the weights in while the MFMAs run.  (Loads
  // into LDS placed between the LDS reads make the compiler wait for nearly all loads in
  // flight before those reads, so they stay in front.)
  constexpr int NW2 = 2 * NF;
  auto compute = [&](int aslot, int bslot, bool spread, int sta, int lslot_n, int stb, int bslot_n) {
    if (spread) {
#pragma unroll
      for (int i = 0; i < AR; ++i) load_one(i, sta, lslot_n, stb, bslot_n);
      // store_a's explicit wait counts on this phase's activation loads being issued
      // before its weight loads: keep the scheduler from moving anything across
      __builtin_amdgcn_sched_barrier(0);
    }
    bf16x8 a[PREFETCH ? 2 : 1][GS];
    if (PREFETCH) {
#pragma unroll
      for (int j = 0; j < GS; ++j) a[0][j] = read_a(aslot, 0, j);
    }
#pragma unroll
    for (int q = 0; q < NG; ++q) {
      const int s = q / (MT / GS), g = q % (MT / GS);
      if (spread) {
#pragma unroll
        for (int i = q * NW2 / NG; i < (q + 1) * NW2 / NG; ++i) load_one(AR + i, sta, lslot_n, stb, bslot_n);
      }
      const int cur = PREFETCH ? (q & 1) : 0;
      if (PREFETCH && q + 1 < NG) {
        const int s1 = (q + 1) / (MT / GS), g1 = (q + 1) % (MT / GS);
        if (g1 * GS < nmf) {
#pragma unroll
          for (int j = 0; j < GS; ++j) a[(q + 1) & 1][j] = read_a(aslot, s1, g1 * GS + j);
        }
      }
      if (g * GS < nmf) {
        if (!PREFETCH) {
#pragma unroll
          for (int j = 0; j < GS; ++j) a[0][j] = read_a(aslot, s, g * GS + j);
        }
#pragma unroll
        for (int j = 0; j < GS; ++j)
#pragma unroll
          for (int nf = 0; nf < NF; ++nf)
            acc[g * GS + j][nf] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[cur][j], rb[bslot][s][nf], acc[g * GS + j][nf], 0, 0, 0);
      }
    }
  };

  // Pipeline.  In the phase of stage st: start the activations of stage st+D and the
  // weights of stage st+WRING-1 (activations first), multiply stage st, make the
  // activations of stage st+1 visible in LDS, barrier.  The memory counter is in issue
  // order, so the wait for stage st+1's activations only covers loads issued up to D-1
  // phases back: later loads stay in flight across it.  Stage s uses weight register
  // slot s mod WRING, activation register slot s mod 2 and LDS slot s mod (D+1).  The
  // phases of the negative stages (loads only) are peeled, so every load is issued
  // inside the pipeline.  The loop is unrolled U times, the least common multiple of the
  // ring lengths, so every slot index is a compile-time constant; each phase tests for
  // the end of K.  (The compiler funnels those exits through one block that also leads
  // back to the loop header, which makes its waits for the weights one phase stricter
  // than needed; a single-exit loop with the last stages peeled measured slower.)
  // Measured: unrolling 3 phases instead of 6 is 1-2.5% faster.
  constexpr int B0 = 1 - WRING;
  constexpr int RA = WRAP ? 2 : 1;           // the register ring only matters on the register path
  constexpr int U0 = WRING * LRING / gcd_c(WRING, LRING);
  constexpr int U = U0 * RA / gcd_c(U0, RA);
  static_assert(U % WRING == 0 && U % LRING == 0 && U % RA == 0, "unroll");
  auto pm = [](int a, int m) { return ((a % m) + m) % m; };
  auto barrier = [&]() {
    if (WRAP) {
      __syncthreads();
    } else {              // the activations' LDS writes were waited for by store_a
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    }
  };
  // Activation loads go to LDS (not the register path) and every phase's loads can be
  // spread over its MFMA groups.
  constexpr bool SPREAD = !WRAP;
  auto phase = [&](int st, int ph) {
    if (SPREAD) {
      compute(pm(ph, LRING), pm(ph, WRING), true, st + D, pm(ph + D, LRING), st + WRING - 1, pm(ph + WRING - 1, WRING));
    } else {
      load_a(st + D, pm(ph + D, 2), pm(ph + D, LRING));
      load_b(st + WRING - 1, pm(ph + WRING - 1, WRING));
      compute(pm(ph, LRING), pm(ph, WRING), false, 0, 0, 0, 0);
    }
    consume_b(pm(ph, WRING));
    store_a(pm(ph + 1, 2), pm(ph + 1, LRING));
    barrier();
  };
  if (nst > 0) {
#pragma unroll
    for (int st = B0; st < 0; ++st) {
      if (st + D >= 0) load_a(st + D, pm(st + D, 2), pm(st + D, LRING));
      __builtin_amdgcn_sched_barrier(0);      // activations before weights (store_a's wait)
      load_b(st + WRING - 1, pm(st + WRING - 1, WRING));
      if (st + 1 >= 0) store_a(pm(st + 1, 2), pm(st + 1, LRING));
      barrier();
    }
    for (int base = 0;; base += U) {
#pragma unroll
      for (int ph = 0; ph < U; ++ph) {
        if (base + ph >= nst) goto pipeline_done;
        phase(base + ph, ph);
      }
    }
  }
pipeline_done:

  // ---- epilogue.  C layout: lane holds rows 4*(lane/16)+v of each 16x16 block, column
  // lane%16; after the quad transpose, row 4*(lane/16) + lane%4 and 4 columns from
  // 4*((lane/4)%4).
  if (!wave_on) return;
  const int qrow = 4 * (lane >> 4) + (lane & 3);
  const int qcol = 4 * ((lane >> 2) & 3);
#pragma unroll
  for (int mf = 0; mf < MT; ++mf) {
    if (mf < nmf) {
      if (PAIRED) {                         // lanes 8..15 of each row group hold the up half
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int r = mf * 16 + 4 * (lane >> 4) + v;
          const float g = acc[mf][0][v];
          const float u = __shfl_xor(g, 8);
          if (r < ti.nrows && (lane & 8) == 0)
            static_cast<uint16_t*>(p.out)[(ti.row_begin + r) * p.N + col_base + (lane & 7)] = f32_to_bf16(silu_f(g) * u);
        }
        continue;
      }
      const int r = mf * 16 + qrow;
      const int64_t orow = ti.row_begin + r;
      if (MODE == MODE_SWIGLU_UP) {
        uint16_t* H = static_cast<uint16_t*>(p.out);
#pragma unroll
        for (int nf = 0; nf < NF / 2; ++nf) {
          float h[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) h[v] = silu_f(acc[mf][nf][v]) * acc[mf][nf + NF / 2][v];
          const u32x2 o = quad_rows_bf16(h, lane);
          if (r < ti.nrows) *reinterpret_cast<u32x2*>(&H[orow * p.N + col_base + nf * 16 + qcol]) = o;
        }
      } else if (MODE == MODE_GELU_UP) {
        uint16_t* H = static_cast<uint16_t*>(p.out);
#pragma unroll
        for (int nf = 0; nf < NF; ++nf) {
          float h[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) h[v] = gelu_f(acc[mf][nf][v]);
          const u32x2 o = quad_rows_bf16(h, lane);
          if (r < ti.nrows) *reinterpret_cast<u32x2*>(&H[orow * p.N + col_base + nf * 16 + qcol]) = o;
        }
      } else {
        float* Y = static_cast<float*>(p.out) + static_cast<int64_t>(ti.split) * p.split_stride;
#pragma unroll
        for (int nf = 0; nf < NF; ++nf) {
          const f32x4 o = quad_rows_f32(acc[mf][nf], lane);
          if (r < ti.nrows) *reinterpret_cast<f32x4*>(&Y[orow * p.N + col_base + nf * 16 + qcol]) = o;
        }
      }
    }
  }
}

template <int MODE, int MT, int NW, bool PK>
__global__ __launch_bounds__(NW * 64, 1) void ffn_gemm_bf16_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) uint16_t As0[MT * 16 * BK];
  __shared__ __attribute__((aligned(16))) uint16_t As1[MT * 16 * BK];
  __shared__ __attribute__((aligned(16))) uint16_t As2[MT * 16 * BK];
  __shared__ __attribute__((aligned(16))) uint16_t As3[ACT_DIST >= 3 ? MT * 16 * BK : 8];
  ffn_gemm_bf16_body<MODE, MT, NW, PK>(p, As0, As1, As2, As3);
}

// ---- wide tile: 256 rows x 256 MFMA columns, 4 waves in a 2 x 2 grid ------------------
// For groups of many rows (the MFMA-bound shapes).  Wave (wm, wn) owns rows 128 wm ..
// 128 wm + 127 and MFMA columns 128 wn .. 128 wn + 127 of the tile: 8 x 8 blocks of
// 16 x 16, so each operand fragment it reads from LDS feeds 8 MFMAs (the 8-wave tile above
// feeds 2 per activation fragment).  Both operands are staged through LDS by
// buffer-to-LDS loads, stored in MFMA fragment order: a 16-row x 32-K fragment is one
// KiB whose 16-byte chunk l is what lane l of the 16x16x32 operand holds (row l % 16,
// K 8 (l / 16) .. +7), so every fragment read is one conflict-free ds_read_b128 and
// no swizzle is needed.  K advances 32 per stage through WS LDS slots of 32 KiB (A and
// B); every wave loads 4 A and 4 B fragments of each stage.  A stage opens with one wait
// (this wave's loads of stage s+1 and its LDS reads of stage s) and one barrier, after
// which slot s+1 is complete and slot s is free; its 64 MFMAs then run in 8 groups (one
// row fragment each), and after each group the wave reads 2 fragments of stage s+1 into
// the other register set and issues 1 load of stage s+WS into slot s.  With one wave per
// SIMD nothing else fills the MFMA pipe while a wave issues memory instructions, so they
// go between the MFMA groups rather than in bursts.  Padding rows of a partial tile get
// an offset past the buffer's range: the load returns zeros without touching memory, and
// their 16-row fragments are not multiplied (one uniform branch per fragment).
constexpr int WIDE_SLOTS = 4;                  // LDS slots (stages in flight: slots - 1)
constexpr int WIDE_UNROLL = 4;                 // stages per loop iteration (a multiple of the slots and of 2)
constexpr int WIDE_FRAG = 512;                 // bf16 elements per 16 x 32 fragment
constexpr int WIDE_READ_GROUPS = 8;            // the next stage's 16 LDS reads go after the first this many MFMA groups

// Wait until at most N vector-memory loads of this wave are outstanding (s_waitcnt
// immediate, gfx9 layout: vmcnt in [3:0] and [15:14]; expcnt and lgkmcnt at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int MODE, bool PK, int WS, int UNR>
__device__ __forceinline__ void ffn_gemm_wide_body(const GemmArgs& p, uint16_t* __restrict__ S0,
                                                   uint16_t* __restrict__ S1, uint16_t* __restrict__ S2,
                                                   uint16_t* __restrict__ S3, uint16_t* __restrict__ S4,
                                                   uint16_t* __restrict__ S5) {
  static_assert(WS >= 3 && WS <= 6 && UNR % WS == 0 && UNR % 2 == 0, "slots and unroll");
  auto slot_ptr = [&](int slot) -> uint16_t* {
    return slot == 0 ? S0 : slot == 1 ? S1 : slot == 2 ? S2 : slot == 3 ? S3 : slot == 4 ? S4 : S5;
  };
  TileInfo ti;
  if (!decode_tile(p, 256, ti)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches and resources
  const int wm = wave >> 1, wn = wave & 1;
  const int nmf = (ti.nrows + 15) >> 4;

  int64_t k_begin = 0, k_end = p.K;
  if (MODE == MODE_DOWN && p.splits > 1) {
    k_begin = static_cast<int64_t>(ti.split) * p.k_chunk;
    k_end = k_begin + p.k_chunk < p.K ? k_begin + p.k_chunk : p.K;
  }
  const int nst = k_end > k_begin ? static_cast<int>((k_end - k_begin) / 32) : 0;

  // ---- A: fragments 4 wave + q of the tile (rows 16 f + lane % 16, K chunk lane / 16)
  const int kc = lane >> 4;
  const int64_t a_row0 = a_base_row(MODE, ti);
  uint32_t aoff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = 16 * (4 * wave + q) + (lane & 15);
    aoff[q] = r < ti.nrows ? static_cast<uint32_t>(((a_source_row(p, MODE, ti.g, ti.row_begin + r) - a_row0) * p.K +
                                                    k_begin + 8 * kc) * 2)
                           : OOB_OFFSET;
  }
  // ---- B: weight-row fragments 4 wave + q of the tile's 256 MFMA columns.  SwiGLU: the
  // columns are [gate u0..u0+63 | up u0..u0+63 | gate u0+64.. | up u0+64..], u0 = 128 ntile,
  // so wave wn's 128 columns hold the gate and up rows of the same 64 hidden units;
  // fragment f = 4 wave + q is a gate fragment for even waves, an up fragment for odd ones.
  const bool shared_grp = ti.g >= p.G;
  const int64_t wstride = shared_grp ? 0 : static_cast<int64_t>(ti.g) * p.N * p.K;
  const uint16_t* W0 = static_cast<const uint16_t*>(shared_grp ? p.sw0 : p.w0) + wstride;
  const uint16_t* W1 = static_cast<const uint16_t*>(shared_grp ? p.sw1 : p.w1) + wstride;
  const uint16_t* Wl = (MODE == MODE_SWIGLU_UP && (wave & 1)) ? W1 : W0;
  uint32_t boff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    int64_t wrow;                              // first weight row of the fragment
    if (MODE == MODE_SWIGLU_UP) wrow = static_cast<int64_t>(ti.ntile) * 128 + 64 * (wave >> 1) + 16 * q;
    else wrow = static_cast<int64_t>(ti.ntile) * 256 + 16 * (4 * wave + q);
    if (wrow >= p.N) wrow = 0;                 // past the last column: a valid row, not stored
    if (PK)
      boff[q] = static_cast<uint32_t>((((wrow >> 4) * (p.K >> 5) + (k_begin >> 5)) * 64 + lane) * 16);
    else
      boff[q] = static_cast<uint32_t>(((wrow + (lane & 15)) * p.K + k_begin + 8 * kc) * 2);
  }
  const __amdgpu_buffer_rsrc_t arsrc = make_rsrc(p.a + a_row0 * p.K);
  const __amdgpu_buffer_rsrc_t brsrc = make_rsrc(Wl);
  constexpr int B_STAGE = PK ? 1024 : 64;      // bytes between the stages of one lane's weight chunk

  // issue every load of stage st (clamped to the last stage: a repeated stage lands in a
  // slot nobody reads again) into LDS slot `slot`: 4 A then 4 B fragments of this wave
  auto issue = [&](int st, int slot) {
    st = st < nst ? st : nst - 1;
    uint16_t* base = slot_ptr(slot);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          arsrc, (__attribute__((address_space(3))) void*)(base + (4 * wave + q) * WIDE_FRAG), 16, aoff[q], st * 64, 0, 0);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          brsrc, (__attribute__((address_space(3))) void*)(base + (16 + 4 * wave + q) * WIDE_FRAG), 16, boff[q],
          st * B_STAGE, 0, 0);
  };
  auto barrier = [&]() {
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  };

  f32x4 acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  bf16x8 ra[2][8], rb[2][8];
  // fragment r of a stage from LDS slot `slot` into register set `buf`: r < 8 the wave's
  // column fragments, r >= 8 its row fragments
  auto read_one = [&](int slot, int buf, int r) {
    const uint16_t* base = slot_ptr(slot);
    if (r < 8) rb[buf][r] = *reinterpret_cast<const bf16x8*>(base + (16 + 8 * wn + r) * WIDE_FRAG + lane * 8);
    else ra[buf][r - 8] = *reinterpret_cast<const bf16x8*>(base + (8 * wm + r - 8) * WIDE_FRAG + lane * 8);
  };
  // One stage (slot and register set are compile-time constants in the unrolled loop).
  // The branches around the MFMA groups also keep the register allocator from mixing the
  // accumulators of different groups (without them it spills).
  auto stage = [&](int st, int slot, int buf) {
    wait_vmcnt<8 * (WS - 2)>();
    __builtin_amdgcn_s_waitcnt(0xc07f);        // lgkmcnt(0), vmcnt and expcnt at their maxima
    barrier();
    __builtin_amdgcn_sched_barrier(0);
    const int ld = st + WS < nst ? st + WS : nst - 1;   // clamped: a repeated stage nobody reads
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (8 * wm + i < nmf) {                  // uniform: row fragment i holds a real row
#pragma unroll
        for (int j = 0; j < 8; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ra[buf][i], rb[buf][j], acc[i][j], 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (r * WIDE_READ_GROUPS / 16 == i) read_one((slot + 1) % WS, buf ^ 1, r);
      uint16_t* base = slot_ptr(slot);
      if (i < 4)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            arsrc, (__attribute__((address_space(3))) void*)(base + (4 * wave + i) * WIDE_FRAG), 16, aoff[i],
            ld * 64, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            brsrc, (__attribute__((address_space(3))) void*)(base + (16 + 4 * wave + i - 4) * WIDE_FRAG), 16,
            boff[i - 4], ld * B_STAGE, 0, 0);
    }
  };
  if (nst > 0) {
#pragma unroll
    for (int st = 0; st < WS; ++st) issue(st, st);
    wait_vmcnt<8 * (WS - 1)>();                // stage 0
    barrier();
#pragma unroll
    for (int r = 0; r < 16; ++r) read_one(0, 0, r);
    for (int base = 0;; base += UNR) {
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        if (base + u >= nst) goto wide_done;
        stage(base + u, u % WS, u & 1);
      }
    }
  }
wide_done:
  wait_vmcnt<0>();                             // no load into this workgroup's LDS outlives it

  // ---- epilogue: C layout, lane holds rows 4 (lane / 16) + v of each 16 x 16 block, column
  // lane % 16; stored through the quad transpose (row 4 (lane / 16) + lane % 4, 4 columns
  // from 4 ((lane / 4) % 4)).  d and F are multiples of 64, so a 16-column block is either
  // inside the output or past it.
  const int qrow = 4 * (lane >> 4) + (lane & 3);
  const int qcol = 4 * ((lane >> 2) & 3);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (8 * wm + i >= nmf) continue;
    const int r = 128 * wm + 16 * i + qrow;
    const int64_t orow = ti.row_begin + r;
    if (MODE == MODE_SWIGLU_UP) {
      uint16_t* H = static_cast<uint16_t*>(p.out);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t u0 = static_cast<int64_t>(ti.ntile) * 128 + 64 * wn + 16 * j;
        if (u0 >= p.N) continue;
        float h[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) h[v] = silu_f(acc[i][j][v]) * acc[i][j + 4][v];
        const u32x2 o = quad_rows_bf16(h, lane);
        if (r < ti.nrows) *reinterpret_cast<u32x2*>(&H[orow * p.N + u0 + qcol]) = o;
      }
    } else if (MODE == MODE_GELU_UP) {
      uint16_t* H = static_cast<uint16_t*>(p.out);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int64_t c0 = static_cast<int64_t>(ti.ntile) * 256 + 128 * wn + 16 * j;
        if (c0 >= p.N) continue;
        float h[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) h[v] = gelu_f(acc[i][j][v]);
        const u32x2 o = quad_rows_bf16(h, lane);
        if (r < ti.nrows) *reinterpret_cast<u32x2*>(&H[orow * p.N + c0 + qcol]) = o;
      }
    } else {
      float* Y = static_cast<float*>(p.out) + static_cast<int64_t>(ti.split) * p.split_stride;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int64_t c0 = static_cast<int64_t>(ti.ntile) * 256 + 128 * wn + 16 * j;
        if (c0 >= p.N) continue;
        const f32x4 o = quad_rows_f32(acc[i][j], lane);
        if (r < ti.nrows) *reinterpret_cast<f32x4*>(&Y[orow * p.N + c0 + qcol]) = o;
      }
    }
  }
}

template <int MODE, bool PK>
__global__ __launch_bounds__(256, 1) void ffn_gemm_wide_kernel(GemmArgs p) {
  // WIDE_SLOTS slots x (16 A + 16 B fragments) x 1 KiB
  // (the slots are disjoint parts of one array, handed to the body as distinct restrict
  // pointers so the compiler can tell the slot being read from the slots being filled)
  constexpr int WS = WIDE_SLOTS;
  constexpr int SLOT = 32 * WIDE_FRAG;
  __shared__ __attribute__((aligned(1024))) uint16_t Sl[WS * SLOT];
  ffn_gemm_wide_body<MODE, PK, WS, WIDE_UNROLL>(p, Sl, Sl + SLOT, Sl + 2 * SLOT, Sl + (WS > 3 ? 3 : 0) * SLOT,
                                                Sl + (WS > 4 ? 4 : 0) * SLOT, Sl + (WS > 5 ? 5 : 0) * SLOT);
}

// Fragment packing of bf16 weights [G, N, K] (K contiguous): 16-byte chunk c of the
// output, with c = ((g * N/16 + i) * K/32 + j) * 64 + l, holds the 8 elements of row
// 16 i + l % 16 at K = 32 j + 8 (l / 16): the 64 lanes of one 16 x 32 MFMA operand
// fragment in lane order.
__global__ __launch_bounds__(256) void pack_weights_kernel(const u32x4* __restrict__ w, u32x4* __restrict__ out,
                                                           int64_t N, int64_t K, int64_t total) {
  const int64_t kb = K >> 5, nb = N >> 4;
  for (int64_t c = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; c < total;
       c += static_cast<int64_t>(gridDim.x) * 256) {
    const int l = static_cast<int>(c & 63);
    const int64_t blk = c >> 6;
    const int64_t j = blk % kb;
    const int64_t gi = blk / kb;              // g * N/16 + i
    const int64_t row = (gi / nb) * N + (gi % nb) * 16 + (l & 15);
    out[c] = w[(row * K + j * 32 + (l >> 4) * 8) >> 3];
  }
}

// ---- fp32 path: 64 x 64 output tile, 256 threads x (4 x 4), K staged 16 at a time.
template <int MODE>
__global__ __launch_bounds__(256) void ffn_gemm_f32_kernel(GemmArgs p) {
  constexpr int TN = 64, TK = 16;
  __shared__ float As[TK][BM_F32 + 1];
  __shared__ float Bs0[TK][TN + 1];
  __shared__ float Bs1[TK][TN + 1];
  TileInfo ti;
  if (!decode_tile(p, BM_F32, ti)) return;
  const int tid = threadIdx.x;
  const int tr = tid / 16, tc = tid % 16;        // 16 x 16 threads, 4 x 4 outputs each
  const bool shared_grp = ti.g >= p.G;
  const float* W0 = static_cast<const float*>(shared_grp ? p.sw0 : p.w0);
  const float* W1 = static_cast<const float*>(shared_grp ? p.sw1 : p.w1);
  const int64_t wstride = shared_grp ? 0 : static_cast<int64_t>(ti.g) * p.N * p.K;
  const int64_t n0 = static_cast<int64_t>(ti.ntile) * TN;
  const float* A = reinterpret_cast<const float*>(p.a);
  float acc0[4][4] = {}, acc1[4][4] = {};
  // loader mapping: 64 rows x 16 k = 1024 values, 4 per thread
  for (int64_t k0 = 0; k0 < p.K; k0 += TK) {
    for (int i = tid; i < BM_F32 * TK; i += 256) {
      const int r = i / TK, kk = i % TK;
      float v = 0.f;
      if (r < ti.nrows && k0 + kk < p.K)
        v = A[a_source_row(p, MODE, ti.g, ti.row_begin + r) * p.K + k0 + kk];
      As[kk][r] = v;
      const int64_t n = n0 + r;
      float b0 = 0.f, b1 = 0.f;
      if (n < p.N && k0 + kk < p.K) {
        b0 = W0[wstride + n * p.K + k0 + kk];
        if (MODE == MODE_SWIGLU_UP) b1 = W1[wstride + n * p.K + k0 + kk];
      }
      Bs0[kk][r] = b0;
      Bs1[kk][r] = b1;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < TK; ++kk) {
      float a[4], b0[4], b1[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { a[i] = As[kk][tr * 4 + i]; b0[i] = Bs0[kk][tc * 4 + i]; b1[i] = Bs1[kk][tc * 4 + i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc0[i][j] = fmaf(a[i], b0[j], acc0[i][j]);
          if (MODE == MODE_SWIGLU_UP) acc1[i][j] = fmaf(a[i], b1[j], acc1[i][j]);
        }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = tr * 4 + i;
    if (r >= ti.nrows) continue;
    const int64_t orow = ti.row_begin + r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t n = n0 + tc * 4 + j;
      if (n >= p.N) continue;
      float v;
      if (MODE == MODE_SWIGLU_UP) v = silu_f(acc0[i][j]) * acc1[i][j];
      else if (MODE == MODE_GELU_UP) v = gelu_f(acc0[i][j]);
      else v = acc0[i][j];
      static_cast<float*>(p.out)[orow * p.N + n] = v;
    }
  }
}

// Sum the split-K partial buffers into y for the rows that belong to some group.
__global__ __launch_bounds__(256) void ffn_reduce_splits_kernel(const float* __restrict__ part, int splits,
                                                                int64_t split_stride, const int32_t* __restrict__ offsets,
                                                                int G, int64_t max_rows, int64_t d,
                                                                float* __restrict__ y) {
  int64_t r0 = offsets[0], r1 = offsets[G];
  r0 = r0 < 0 ? 0 : r0;
  r1 = r1 > max_rows ? max_rows : r1;
  const int64_t n4 = d / 4;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < (r1 - r0) * n4;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t r = r0 + i / n4, c = (i % n4) * 4;
    f32x4 s = *reinterpret_cast<const f32x4*>(part + r * d + c);
    for (int sp = 1; sp < splits; ++sp) s += *reinterpret_cast<const f32x4*>(part + sp * split_stride + r * d + c);
    *reinterpret_cast<f32x4*>(y + r * d + c) = s;
  }
}


// Launch one bf16 grouped GEMM with the M-tile (MT*16 rows) chosen by the plan (a shape
// that bf16_tile_supported accepts; the schedule was built for the same height).
template <int MODE, bool PK>
void launch_bf16_gemm_l(int bm, int nw, int64_t grid, const GemmArgs& g, hipStream_t s) {
  const unsigned gr = static_cast<unsigned>(grid);
  if (nw == 16) {
    switch (bm) {
      case 32: ffn_gemm_bf16_kernel<MODE, 2, 16, PK><<<gr, 1024, 0, s>>>(g); break;
      case 64: ffn_gemm_bf16_kernel<MODE, 4, 16, PK><<<gr, 1024, 0, s>>>(g); break;
      case 128: ffn_gemm_bf16_kernel<MODE, 8, 16, PK><<<gr, 1024, 0, s>>>(g); break;
      case 256: ffn_gemm_bf16_kernel<MODE, 16, 16, PK><<<gr, 1024, 0, s>>>(g); break;
      default: break;
    }
  } else if (nw == 8) {
    switch (bm) {
      case 32: ffn_gemm_bf16_kernel<MODE, 2, 8, PK><<<gr, 512, 0, s>>>(g); break;
      case 64: ffn_gemm_bf16_kernel<MODE, 4, 8, PK><<<gr, 512, 0, s>>>(g); break;
      case 128: ffn_gemm_bf16_kernel<MODE, 8, 8, PK><<<gr, 512, 0, s>>>(g); break;
      case 192: ffn_gemm_bf16_kernel<MODE, 12, 8, PK><<<gr, 512, 0, s>>>(g); break;
      case 256: ffn_gemm_bf16_kernel<MODE, 16, 8, PK><<<gr, 512, 0, s>>>(g); break;
      default: break;
    }
  } else {
    switch (bm) {
      case 32: ffn_gemm_bf16_kernel<MODE, 2, 4, PK><<<gr, 256, 0, s>>>(g); break;
      case 64: ffn_gemm_bf16_kernel<MODE, 4, 4, PK><<<gr, 256, 0, s>>>(g); break;
      case 128: ffn_gemm_bf16_kernel<MODE, 8, 4, PK><<<gr, 256, 0, s>>>(g); break;
      case 256: ffn_gemm_wide_kernel<MODE, PK><<<gr, 256, 0, s>>>(g); break;   // 2 x 2 waves
      default: break;
    }
  }
}

template <int MODE>
void launch_bf16_gemm(bool packed, int bm, int nw, int64_t grid, const GemmArgs& g, hipStream_t s) {
  if (packed) launch_bf16_gemm_l<MODE, true>(bm, nw, grid, g, s);
  else launch_bf16_gemm_l<MODE, false>(bm, nw, grid, g, s);
}

}  // namespace

// Tile shapes with a bf16 kernel: 32, 64, 128 or 256 rows with 4, 8 or 16 waves, and 192
// rows with 8 waves (12 row fragments; at 4 or 16 waves that height would need the register
// path for the activations or more registers than a wave has).
bool bf16_tile_supported(int bm, int nw) {
  if (nw != 4 && nw != 8 && nw != 16) return false;
  return bm == 32 || bm == 64 || bm == 128 || bm == 256 || (bm == 192 && nw == 8);
}

// M-tile height: the smallest of 32/64/128/192/256 rows that holds a typical routed group
// in one tile, so each expert's weights stream once.  The rows per group are only known on
// the device; the host estimate is the capacity when one is set, else 1.6x the mean load
// (plus a margin for small loads).  192 rows are taken up to an estimate of 224: the
// activation loads of a tile cover its full height (padding rows included), and a group
// over 192 rows costs a second, mostly empty tile whose weights come from L2, which pays
// while such groups are rare (measured on 64 experts x 128 rows on average: 2% faster
// than 256-row tiles).  A shared group (T rows) does not raise it: its M-tiles are
// adjacent in the schedule and share its weights in L2, while routed experts are the
// bulk of the weight bytes.
FfnPlan ffn_plan(int64_t max_rows, int G, int64_t shared_rows, int64_t d, int64_t F, int act, int dt,
                 int64_t capacity, int tile_rows, int tile_waves) {
  FfnPlan pl{};
  (void)act;
  const bool has_shared = shared_rows > 0;
  const int Gt = G + (has_shared ? 1 : 0);
  if (dt == MOE_BF16) {
    const int64_t routed = max_rows - (has_shared ? shared_rows : 0);
    double est = 1.6 * static_cast<double>(routed) / (G > 0 ? G : 1) + 16.0;
    if (capacity > 0 && static_cast<double>(capacity) < est) est = static_cast<double>(capacity);
    pl.bm = est <= 32 ? 32 : est <= 64 ? 64 : est <= 128 ? 128 : est <= 224 ? 192 : BM;
    pl.nw = 8;
    // the caller's explicit tile shape (moe_tile_t), already checked against the kernels
    if (tile_waves > 0) pl.nw = tile_waves;
    if (tile_rows > 0) pl.bm = tile_rows;
    if (!bf16_tile_supported(pl.bm, pl.nw)) pl.bm = BM;     // waves alone: 192 rows need 8
  } else {
    pl.bm = BM_F32;
  }
  pl.max_mtiles = (max_rows + pl.bm - 1) / pl.bm + Gt + 1;
  pl.splits = 1;
  if (dt == MOE_BF16) {
    const int64_t nt2 = (d + 255) / 256;
    int64_t est = (max_rows + pl.bm - 1) / pl.bm;
    const int64_t busy = G < max_rows ? G : max_rows;
    if (busy > est) est = busy;
    // split the down projection over K only until there is about one tile per CU: each
    // split writes fp32 partial sums that the combine reads back (measured with packed
    // weights: decode T=1..4 fastest at 256 tiles; T=16 and capacity-e16 unsplit)
    while (est * nt2 * pl.splits < 256 && F / (BK * pl.splits * 2) >= 8) pl.splits *= 2;
  }
  const size_t elem = dt == MOE_BF16 ? 2 : 4;
  size_t ws = align_up(sched_words(Gt, pl.max_mtiles) * sizeof(int32_t), 256);
  ws += align_up(static_cast<size_t>(max_rows) * F * elem, 256);                       // H
  if (pl.splits > 1) ws += align_up(static_cast<size_t>(pl.splits) * max_rows * d * 4, 256);  // partials
  pl.ws_bytes = ws;
  return pl;
}

moe_status_t launch_ffn(const FfnProblem& p, const FfnPlan& plan, float* y, bool reduce_splits,
                        void* ws, hipStream_t s, void* const* ev) {
  auto mark = [&](int i) {
    if (ev) (void)hipEventRecord(static_cast<hipEvent_t>(ev[i]), s);
  };
  const bool has_shared = p.shared_rows > 0;
  const int Gt = p.G + (has_shared ? 1 : 0);
  const bool bf = p.dt == MOE_BF16;
  const bool packed = p.layout == MOE_LAYOUT_PACKED;
  const int bm = plan.bm;
  WsCarver c(ws);
  int32_t* sched = c.take<int32_t>(sched_words(Gt, plan.max_mtiles));
  void* H = bf ? static_cast<void*>(c.take<uint16_t>(static_cast<size_t>(p.max_rows) * p.F))
               : static_cast<void*>(c.take<float>(static_cast<size_t>(p.max_rows) * p.F));
  float* part = nullptr;
  if (plan.splits > 1) part = c.take<float>(static_cast<size_t>(plan.splits) * p.max_rows * p.d);
  if (Gt == 0 || p.max_rows == 0) {
    mark(0); mark(1); mark(2);
    return MOE_OK;
  }
  if (bf && !bf16_tile_supported(bm, plan.nw)) return MOE_EINVAL;

  ffn_schedule_kernel<<<1, 1024, 0, s>>>(p.offsets, p.G, p.max_rows, p.shared_rows, p.shared_row0, bm,
                                         plan.max_mtiles, sched);
  if (moe_status_t st = check_launch("ffn schedule kernel")) return st;
  mark(0);

  GemmArgs g{};
  g.perm = p.perm;
  g.k_div = p.k > 0 ? p.k : 1;
  g.sched = sched;
  g.max_mtiles = plan.max_mtiles;
  g.G = p.G;
  g.Gt = Gt;
  g.shared_row0 = p.shared_row0;
  g.splits = 1;
  g.split_stride = 0;

  // ---- up projection: H = act(x W_gate^T) [* (x W_up^T)]
  const bool swiglu = p.act == MOE_ACT_SWIGLU;
  g.a = static_cast<const uint16_t*>(p.x);
  g.w0 = p.w_gate;
  g.w1 = swiglu ? p.w_up : nullptr;
  g.sw0 = p.s_gate;
  g.sw1 = swiglu ? p.s_up : nullptr;
  g.K = p.d;
  g.N = p.F;
  g.k_chunk = p.d;
  g.out = H;
  if (bf) {
    g.nt = static_cast<int>(swiglu ? (p.F + 127) / 128 : (p.F + 255) / 256);
    const int64_t grid = ((plan.max_mtiles * g.nt + 7) / 8) * 8;
    if (swiglu) launch_bf16_gemm<MODE_SWIGLU_UP>(packed, bm, plan.nw, grid, g, s);
    else launch_bf16_gemm<MODE_GELU_UP>(packed, bm, plan.nw, grid, g, s);
  } else {
    g.nt = static_cast<int>((p.F + 63) / 64);
    const int64_t grid = ((plan.max_mtiles * g.nt + 7) / 8) * 8;
    if (swiglu) ffn_gemm_f32_kernel<MODE_SWIGLU_UP><<<static_cast<unsigned>(grid), 256, 0, s>>>(g);
    else ffn_gemm_f32_kernel<MODE_GELU_UP><<<static_cast<unsigned>(grid), 256, 0, s>>>(g);
  }
  if (moe_status_t st = check_launch("ffn up-projection kernel")) return st;
  mark(1);

  // ---- down projection: y = H W_down^T
  g.a = static_cast<const uint16_t*>(H);
  g.perm = nullptr;
  g.w0 = p.w_down;
  g.w1 = nullptr;
  g.sw0 = p.s_down;
  g.sw1 = nullptr;
  g.K = p.F;
  g.N = p.d;
  if (bf) {
    g.nt = static_cast<int>((p.d + 255) / 256);
    g.splits = plan.splits;
    g.k_chunk = ((p.F / BK + plan.splits - 1) / plan.splits) * BK;
    g.split_stride = p.max_rows * p.d;
    g.out = plan.splits > 1 && reduce_splits ? static_cast<void*>(part) : static_cast<void*>(y);
    const int64_t grid = ((plan.max_mtiles * g.nt * g.splits + 7) / 8) * 8;
    launch_bf16_gemm<MODE_DOWN>(packed, bm, plan.nw, grid, g, s);
  } else {
    g.nt = static_cast<int>((p.d + 63) / 64);
    g.k_chunk = p.F;
    g.out = y;
    const int64_t grid = ((plan.max_mtiles * g.nt + 7) / 8) * 8;
    ffn_gemm_f32_kernel<MODE_DOWN><<<static_cast<unsigned>(grid), 256, 0, s>>>(g);
  }
  if (moe_status_t st = check_launch("ffn down-projection kernel")) return st;
  mark(2);

  if (bf && plan.splits > 1 && reduce_splits) {
    ffn_reduce_splits_kernel<<<1024, 256, 0, s>>>(part, plan.splits, p.max_rows * p.d, p.offsets, p.G,
                                                   p.max_rows, p.d, y);
    if (moe_status_t st = check_launch("ffn split reduction kernel")) return st;
  }
  return MOE_OK;
}

moe_status_t launch_pack(const void* w, void* packed, int64_t G, int64_t N, int64_t K, hipStream_t s) {
  const int64_t total = G * N * K / 8;
  const int64_t want = (total + 255) / 256;
  const unsigned grid = static_cast<unsigned>(want < 8192 ? want : 8192);
  pack_weights_kernel<<<grid, 256, 0, s>>>(static_cast<const u32x4*>(w), static_cast<u32x4*>(packed), N, K, total);
  return check_launch("weight packing kernel");
}

}  // namespace moe
